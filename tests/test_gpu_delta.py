"""GPU parity of the delta-rule state scan (DeltaNet shapes, including
head_k_dim != head_v_dim) against the sequential fp64 oracle, through the C ABI.

Tolerance: normwise relative error <= 2e-3 per (batch, head) slice of o and of
s_final (bf16 inputs, fp32 state).  K != V cases are included because a
product taken on the wrong side of S only shows there [SunnyNet log §4.2].
"""
import numpy as np
import pytest
import torch

import oracle
from linear_recurrence_scan_fma_amd import binding, inputs
from _helpers import dev, rel_heads, say

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = binding.Context(0)
    yield c
    c.close()


def _gpu(ctx, d, s0=None):
    o, fin = binding.scan_delta(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["beta"]), d["scale"],
                                dev(s0))
    torch.cuda.synchronize()
    return o, fin


def _ref(d, s0=None):
    return oracle.scan_delta(d["q"], d["k"], d["v"], d["beta"], d["scale"], s0)


def _check(ctx, d, s0=None):
    o, fin = _gpu(ctx, d, s0)
    ro, rf = _ref(d, s0)
    eo, ef = rel_heads(o, ro, "bthv"), rel_heads(fin, rf, "bhkv")
    say(f"   rel err o={eo:.2e} s_final={ef:.2e}")
    assert eo <= TOL and ef <= TOL, (eo, ef)


@pytest.mark.parametrize("shape", [
    (2, 200, 3, 128, 128),   # DeltaNet head shape, ragged T
    (1, 64, 2, 128, 128),    # one chunk
    (2, 150, 2, 64, 128),    # K = 64 != V = 128
    (1, 100, 2, 128, 64),    # K > V
    (1, 130, 2, 128, 40),    # ragged V tile
    (1, 77, 2, 36, 20),      # K, V not multiples of 8 (scalar loads)
    (1, 1, 1, 128, 128),     # T = 1
    (2, 50, 2, 1, 1),        # K = V = 1
], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_s0", [False, True])
def test_delta_parity(ctx, shape, with_s0):
    B, T, H, K, V = shape
    say(f"delta {shape} s0={with_s0}")
    d = inputs.deltanet(B=B, T=T, H=H, K=K, V=V, seed=300 + T + K)
    s0 = inputs.random_state((B, H, K, V), 8) if with_s0 else None
    _check(ctx, d, s0)


def test_delta_readout_scale_and_unnormalised_keys(ctx):
    # keys a little longer than unit norm and a readout scale: the chunked form
    # is exact algebra, so it must track the recurrence for any such input
    B, T, H, K, V = 1, 190, 2, 64, 96
    d = inputs.deltanet(B=B, T=T, H=H, K=K, V=V, seed=77)
    d["k"] = (d["k"].float() * 1.2).to(torch.bfloat16)
    d["scale"] = 0.125
    _check(ctx, d, inputs.random_state((B, H, K, V), 9))


def test_delta_beta_extremes(ctx):
    # beta = 0 keeps the state; beta = 1 with unit keys overwrites the read-back
    B, T, H, K, V = 1, 130, 2, 128, 64
    d = inputs.deltanet(B=B, T=T, H=H, K=K, V=V, seed=78)
    d["beta"] = torch.zeros_like(d["beta"])
    _check(ctx, d, inputs.random_state((B, H, K, V), 10))
    d["beta"] = torch.ones_like(d["beta"])
    _check(ctx, d, inputs.random_state((B, H, K, V), 11))


def test_continuation(ctx):
    B, T, H, K, V = 1, 260, 2, 128, 128
    d = inputs.deltanet(B=B, T=T, H=H, K=K, V=V, seed=79)
    s0 = inputs.random_state((B, H, K, V), 12)
    o_full, f_full = _gpu(ctx, d, s0)
    seq = ("q", "k", "v", "beta")
    for t1 in (1, 37, 64, 130):
        first = {n: (x[:, :t1] if n in seq else x) for n, x in d.items()}
        second = {n: (x[:, t1:] if n in seq else x) for n, x in d.items()}
        o1, f1 = _gpu(ctx, first, s0)
        o2, f2 = _gpu(ctx, second, f1.cpu())
        assert rel_heads(torch.cat([o1, o2], 1), o_full, "bthv") <= 1e-4
        assert rel_heads(f2, f_full, "bhkv") <= 1e-4


def test_workspace_regrowth_between_calls(ctx):
    # the context's per-chunk scratch grows with B*H*T; interleave sizes
    for i, (B, T, H) in enumerate([(1, 70, 1), (2, 400, 3), (1, 65, 2), (1, 900, 2)]):
        d = inputs.deltanet(B=B, T=T, H=H, K=64, V=64, seed=400 + i)
        _check(ctx, d)


def test_rejects_bad_arguments(ctx):
    d = inputs.deltanet(B=1, T=8, H=2, K=16, V=16, seed=1)
    q, k, v, beta = (dev(d[n]) for n in ("q", "k", "v", "beta"))
    o = torch.empty((1, 8, 2, 16), device="cuda:0")
    f = torch.empty((1, 2, 16, 16), device="cuda:0")
    L = binding.lib()
    P = lambda t: t.data_ptr()  # noqa: E731
    assert L.lrs_scan_delta(ctx.handle, P(q), P(k), P(v), P(beta), 1.0, None, P(o), P(f),
                            1, 8, 2, 16, 0, None) == binding.LRS_E_INVAL          # V = 0
    assert L.lrs_scan_delta(ctx.handle, P(q), P(k), P(v), P(beta), 1.0, None, P(o), P(f),
                            1, 8, 2, 256, 16, None) == binding.LRS_E_UNSUPPORTED  # K > 128
    assert L.lrs_scan_delta(ctx.handle, P(q), P(k), P(v), P(beta), 1.0, None, P(o), P(o),
                            1, 8, 2, 16, 16, None) == binding.LRS_E_INVAL         # outputs alias
    assert L.lrs_scan_delta(None, P(q), P(k), P(v), P(beta), 1.0, None, P(o), P(f),
                            1, 8, 2, 16, 16, None) == binding.LRS_E_INVAL


@pytest.mark.parametrize("cfg", ["k128", "k64"])
def test_deltanet_full_size_sampled(ctx, cfg):
    shape = inputs.DELTANET if cfg == "k128" else inputs.DELTANET_K64
    say(f"delta full size {shape}")
    d = inputs.deltanet(**shape)
    o, fin = _gpu(ctx, d)
    for b, h in [(0, 0), (3, 7), (1, 4)]:
        sub = {n: (x[b:b + 1, :, h:h + 1] if n in ("q", "k", "v", "beta") else x) for n, x in d.items()}
        ro, rf = _ref(sub)
        eo = rel_heads(o[b:b + 1, :, h:h + 1], ro, "bthv")
        ef = rel_heads(fin[b:b + 1, h:h + 1], rf, "bhkv")
        say(f"   head ({b},{h}): rel err o={eo:.2e} s_final={ef:.2e}")
        assert eo <= TOL and ef <= TOL
    assert torch.isfinite(o).all() and torch.isfinite(fin).all()
