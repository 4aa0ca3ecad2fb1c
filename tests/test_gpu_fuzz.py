"""Seeded random-shape parity sweep of every matrix-state scan against the
fp64 oracle, through the C ABI: odd and ragged K, V and T, several heads and
groups, with and without an initial state, and a random time-segment count
(decay-separable scans and delta rule alike; the delta rule also in its
decayed form at keys up to 128 wide).  Each case prints its shape before it
runs.

Tolerance as in the per-scan tests: normwise relative error <= 2e-3 per
(batch, head) slice of o and of s_final.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_recurrence_scan_fma_amd import binding, inputs
from _helpers import dev, rel_heads, say

pytestmark = pytest.mark.gpu

TOL = 2e-3
CASES = 10


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = binding.Context(0)
    yield c
    c.close()


def _shape(rng, kmax):
    B = int(rng.integers(1, 3))
    T = int(rng.choice([1, 63, 64, 65, int(rng.integers(2, 400))]))
    H = int(rng.integers(1, 4))
    K = int(rng.choice([kmax, int(rng.integers(1, kmax + 1))]))
    V = int(rng.choice([64, 128, int(rng.integers(1, 161))]))
    return B, T, H, K, V


def _assert(name, o, fin, ro, rf):
    eo, ef = rel_heads(o, ro, "bthv"), rel_heads(fin, rf, "bhkv")
    say(f"   {name}: rel err o={eo:.2e} s_final={ef:.2e}")
    assert eo <= TOL and ef <= TOL, (eo, ef)


class _Segments:
    def __init__(self, ctx, n, param=binding.LRS_PARAM_DIAG_SEGMENTS):
        self.ctx, self.n, self.param = ctx, n, param

    def __enter__(self):
        binding.lrs_context_set_param(self.ctx, self.param, self.n)

    def __exit__(self, *exc):
        binding.lrs_context_set_param(self.ctx, self.param, 0)


@pytest.mark.parametrize("case", range(CASES))
@pytest.mark.parametrize("family", ["mamba2", "gla", "assoc"])
def test_diag_outer_random_shapes(ctx, family, case):
    rng = np.random.default_rng(1000 * ["mamba2", "gla", "assoc"].index(family) + case)
    B, T, H, K, V = _shape(rng, 128 if family != "assoc" else 64)
    seed = int(rng.integers(1 << 30))
    segments = int(rng.choice([0, 1, 2, 3, 5, 9]))
    with_s0 = bool(rng.integers(2))
    say(f"diag {family} B={B} T={T} H={H} K={K} V={V} segments={segments} s0={with_s0} seed={seed}")
    s0 = inputs.random_state((B, H, K, V), seed + 1) if with_s0 else None
    with _Segments(ctx, segments):
        if family == "mamba2":
            d = inputs.mamba2(B=B, T=T, H=H, K=K, V=V, seed=seed)
            o, fin = binding.scan_diag_outer(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]), 0,
                                             dev(d["k_scale"]), d["scale"], dev(s0))
            ro, rf = oracle.scan_diag_outer(d["q"], d["k"], d["v"], d["g"], 0, d["k_scale"], d["scale"], s0)
        elif family == "gla":
            d = inputs.gla(B=B, T=T, H=H, K=K, V=V, seed=seed)
            o, fin = binding.scan_diag_outer(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]), 1, None,
                                             d["scale"], dev(s0))
            ro, rf = oracle.scan_diag_outer(d["q"], d["k"], d["v"], d["g"], 1, None, d["scale"], s0)
        else:
            d = inputs.assoc_memory(B=B, T=T, H=H, K=K, V=V, seed=seed)
            o, fin = binding.scan_diag_outer_keyscale(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]),
                                                      dev(d["k_scale_key"]), d["scale"], dev(s0))
            ro, rf = oracle.scan_diag_outer(d["q"], d["k"], d["v"], d["g"], 1, None, d["scale"], s0,
                                            k_scale_key=d["k_scale_key"])
        torch.cuda.synchronize()
    _assert(family, o, fin, ro, rf)


DELTA_FAMILIES = ["deltanet", "rwkv7", "decay_k128"]


@pytest.mark.parametrize("case", range(CASES))
@pytest.mark.parametrize("family", DELTA_FAMILIES)
def test_delta_random_shapes(ctx, family, case):
    # decay_k128: the decayed form with keys up to 128 wide; every family also
    # draws a time-segment count (0: automatic)
    rng = np.random.default_rng(5000 + 1000 * DELTA_FAMILIES.index(family) + case)
    B, T, H, K, V = _shape(rng, 64 if family == "rwkv7" else 128)
    seed = int(rng.integers(1 << 30))
    with_s0 = bool(rng.integers(2))
    segments = int(rng.choice([0, 1, 2, 3, 5]))
    say(f"delta {family} B={B} T={T} H={H} K={K} V={V} s0={with_s0} segments={segments} seed={seed}")
    s0 = inputs.random_state((B, H, K, V), seed + 1, std=0.3) if with_s0 else None
    with _Segments(ctx, segments, binding.LRS_PARAM_DELTA_SEGMENTS):
        if family == "deltanet":
            d = inputs.deltanet(B=B, T=T, H=H, K=K, V=V, seed=seed)
            o, fin = binding.scan_delta(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["beta"]), d["scale"],
                                        dev(s0))
            ro, rf = oracle.scan_delta(d["q"], d["k"], d["v"], d["beta"], d["scale"], s0)
        else:
            d = inputs.rwkv7(B=B, T=T, H=H, K=K, V=V, seed=seed)
            o, fin = binding.scan_delta_decay(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]),
                                              dev(d["beta"]), d["scale"], dev(s0))
            ro, rf = oracle.scan_delta_decay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], s0)
        torch.cuda.synchronize()
    _assert(family, o, fin, ro, rf)
