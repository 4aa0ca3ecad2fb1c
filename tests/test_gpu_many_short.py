"""GPU parity on many short sequences (a serving-like batch: B = 96, T = 40,
one partial chunk each; and B = 48, T = 130, three chunks with a ragged
tail) for every matrix scan, against the sequential fp64 oracle, through the
C ABI.  Here the grids are wide (thousands of workgroups), every call takes
the one-segment plan, and most chunks are partial.

Tolerance as in the per-scan tests: 2e-3 normwise per (batch, head) slice.
"""
import pytest
import torch

import oracle
from linear_recurrence_scan_fma_amd import binding, inputs
from _helpers import dev, rel_heads, say

pytestmark = pytest.mark.gpu

TOL = 2e-3
SHAPES = [(96, 40), (48, 130)]


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = binding.Context(0)
    yield c
    c.close()


def _check(name, o, fin, ro, rf):
    eo, ef = rel_heads(o, ro, "bthv"), rel_heads(fin, rf, "bhkv")
    say(f"   {name}: rel err o={eo:.2e} s_final={ef:.2e}")
    assert eo <= TOL and ef <= TOL, (eo, ef)


@pytest.mark.parametrize("B,T", SHAPES)
@pytest.mark.parametrize("family", ["deltanet", "rwkv7"])
def test_delta_many_short(ctx, family, B, T):
    K = V = 128 if family == "deltanet" else 64
    H = 4
    say(f"delta {family} B={B} T={T} H={H} K={K} V={V}")
    s0 = inputs.random_state((B, H, K, V), 81, std=0.3)
    if family == "deltanet":
        d = inputs.deltanet(B=B, T=T, H=H, K=K, V=V, seed=801 + T)
        o, fin = binding.scan_delta(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["beta"]), d["scale"], dev(s0))
        torch.cuda.synchronize()
        ro, rf = oracle.scan_delta(d["q"], d["k"], d["v"], d["beta"], d["scale"], s0)
    else:
        d = inputs.rwkv7(B=B, T=T, H=H, K=K, V=V, seed=802 + T)
        o, fin = binding.scan_delta_decay(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]), dev(d["beta"]),
                                          d["scale"], dev(s0))
        torch.cuda.synchronize()
        ro, rf = oracle.scan_delta_decay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], s0)
    _check(family, o, fin, ro, rf)


@pytest.mark.parametrize("B,T", SHAPES)
@pytest.mark.parametrize("family", ["gla", "mamba2"])
def test_diag_outer_many_short(ctx, family, B, T):
    say(f"diag {family} B={B} T={T}")
    if family == "gla":
        d = inputs.gla(B=B, T=T, H=4, K=128, V=128, seed=803 + T)
    else:
        d = inputs.mamba2(B=B, T=T, H=8, K=128, V=64, seed=804 + T)
    H, K, V = d["v"].shape[2], d["k"].shape[3], d["v"].shape[3]
    s0 = inputs.random_state((B, H, K, V), 83)
    o, fin = binding.scan_diag_outer(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]), d["decay_mode"],
                                     dev(d["k_scale"]), d["scale"], dev(s0))
    torch.cuda.synchronize()
    ro, rf = oracle.scan_diag_outer(d["q"], d["k"], d["v"], d["g"], d["decay_mode"], d["k_scale"], d["scale"], s0)
    _check(family, o, fin, ro, rf)
