"""GPU parity of the delta rule with a per-key decay (RWKV-7's state update
[SunnyNet log §5.1], key-major with an in-context rate beta) against the
sequential fp64 oracle, through the C ABI.

Tolerance: normwise relative error <= 2e-3 per (batch, head) slice of o and of
s_final, as for the other matrix scans.  Cases cover both key widths of the
kernel (K <= 64 and 64 < K <= 128), K != V both ways, ragged chunks and V
tiles, the scalar-load path, T = 1, K = V = 1, decays strong enough to take
the kernel's exact-exponential path, growth (g > 0), the no-decay limit, and
the full-size workload at K = V = 128 on every head with both paths present.
"""
import pytest
import torch

import oracle
from linear_recurrence_scan_fma_amd import binding, inputs
from _helpers import dev, rel_heads, say

pytestmark = pytest.mark.gpu

TOL = 2e-3
SEQ = ("q", "k", "v", "beta", "g")


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = binding.Context(0)
    yield c
    c.close()


def _gpu(ctx, d, s0=None):
    o, fin = binding.scan_delta_decay(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]),
                                      dev(d["beta"]), d["scale"], dev(s0))
    torch.cuda.synchronize()
    return o, fin


def _ref(d, s0=None):
    return oracle.scan_delta_decay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], s0)


def _check(ctx, d, s0=None, tol=TOL):
    o, fin = _gpu(ctx, d, s0)
    ro, rf = _ref(d, s0)
    eo, ef = rel_heads(o, ro, "bthv"), rel_heads(fin, rf, "bhkv")
    say(f"   rel err o={eo:.2e} s_final={ef:.2e}")
    assert eo <= tol and ef <= tol, (eo, ef)


@pytest.mark.parametrize("shape", [
    (2, 200, 3, 64, 64),     # RWKV-7 head shape, ragged T
    (1, 64, 2, 64, 64),      # one chunk
    (2, 150, 2, 64, 128),    # K < V
    (1, 100, 2, 64, 32),     # K > V
    (1, 130, 2, 48, 40),     # K < 64 (zero-padded keys), ragged V tile
    (1, 77, 2, 36, 20),      # K, V not multiples of 8 (scalar loads)
    (1, 1, 1, 64, 64),       # T = 1
    (2, 50, 2, 1, 1),        # K = V = 1
    (2, 200, 3, 128, 128),   # K = 128: DeltaNet's head shape, ragged T
    (1, 150, 2, 128, 64),    # K = 128 > V
    (1, 130, 2, 100, 40),    # 64 < K < 128 (zero-padded keys), ragged V tile
    (1, 77, 2, 90, 20),      # 64 < K, not a multiple of 8 (scalar loads)
    (1, 1, 1, 128, 128),     # K = 128, T = 1
], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_s0", [False, True])
def test_delta_decay_parity(ctx, shape, with_s0):
    B, T, H, K, V = shape
    say(f"delta decay {shape} s0={with_s0}")
    d = inputs.rwkv7(B=B, T=T, H=H, K=K, V=V, seed=500 + T + K)
    s0 = inputs.random_state((B, H, K, V), 13) if with_s0 else None
    _check(ctx, d, s0)


@pytest.mark.parametrize("K", [64, 128])
@pytest.mark.parametrize("gval", [-2.0, -0.9], ids=["all_exact_path", "mixed"])
def test_delta_decay_strong_decay(ctx, gval, K):
    # -2 nats per step: every chunk's running sum spans 126 nats (exact-exponential
    # path); -0.9 on every other step: spans near the switch, both paths
    B, T, H, V = 1, 260, 2, 64
    say(f"delta decay strong g={gval} K={K}")
    d = inputs.rwkv7(B=B, T=T, H=H, K=K, V=V, seed=81)
    g = d["g"].clone()
    if gval == -2.0:
        g[:] = -2.0
    else:
        g[:, ::2] = -0.9
        g[:, :, :, : K // 2] *= 1.5
    d["g"] = g
    _check(ctx, d, inputs.random_state((B, H, K, V), 14))


def test_delta_decay_growth_and_no_decay(ctx):
    B, T, H, K, V = 1, 190, 2, 64, 48
    d = inputs.rwkv7(B=B, T=T, H=H, K=K, V=V, seed=82)
    s0 = inputs.random_state((B, H, K, V), 15)
    d["g"] = torch.full_like(d["g"], 0.004)   # a slowly growing state
    _check(ctx, d, s0)
    d["g"] = torch.zeros_like(d["g"])         # no decay: the plain delta rule
    _check(ctx, d, s0)
    o1, f1 = _gpu(ctx, d, s0)
    o2, f2 = binding.scan_delta(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["beta"]), d["scale"],
                                dev(s0))
    assert rel_heads(o1, o2, "bthv") <= 1e-4 and rel_heads(f1, f2, "bhkv") <= 1e-4


def test_delta_decay_readout_scale_and_beta_extremes(ctx):
    B, T, H, K, V = 1, 130, 2, 64, 64
    d = inputs.rwkv7(B=B, T=T, H=H, K=K, V=V, seed=83)
    d["scale"] = 0.125
    d["beta"] = torch.zeros_like(d["beta"])   # pure decay of the initial state
    _check(ctx, d, inputs.random_state((B, H, K, V), 16))
    d["beta"] = torch.ones_like(d["beta"])    # the page's form (no in-context rate)
    _check(ctx, d, inputs.random_state((B, H, K, V), 17))


def test_delta_decay_continuation(ctx):
    B, T, H, K, V = 1, 260, 2, 64, 64
    d = inputs.rwkv7(B=B, T=T, H=H, K=K, V=V, seed=84)
    s0 = inputs.random_state((B, H, K, V), 18)
    o_full, f_full = _gpu(ctx, d, s0)
    for t1 in (1, 37, 64, 130):
        first = {n: (x[:, :t1] if n in SEQ else x) for n, x in d.items()}
        second = {n: (x[:, t1:] if n in SEQ else x) for n, x in d.items()}
        o1, f1 = _gpu(ctx, first, s0)
        o2, f2 = _gpu(ctx, second, f1.cpu())
        assert rel_heads(torch.cat([o1, o2], 1), o_full, "bthv") <= 1e-4
        assert rel_heads(f2, f_full, "bhkv") <= 1e-4


def test_delta_decay_shares_workspace_with_plain_form(ctx):
    # the two forms use one context workspace with different chunk blocks;
    # interleave them and their sizes
    for i, (B, T, H) in enumerate([(1, 70, 1), (2, 400, 3), (1, 65, 2), (1, 900, 2)]):
        d = inputs.rwkv7(B=B, T=T, H=H, K=64, V=64, seed=600 + i)
        _check(ctx, d)
        dn = inputs.deltanet(B=B, T=T, H=H, K=128, V=64, seed=700 + i)
        o, fin = binding.scan_delta(ctx, dev(dn["q"]), dev(dn["k"]), dev(dn["v"]), dev(dn["beta"]), 1.0)
        torch.cuda.synchronize()
        ro, rf = oracle.scan_delta(dn["q"], dn["k"], dn["v"], dn["beta"], 1.0)
        assert rel_heads(o, ro, "bthv") <= TOL and rel_heads(fin, rf, "bhkv") <= TOL


def test_delta_decay_rejects_bad_arguments(ctx):
    d = inputs.rwkv7(B=1, T=8, H=2, K=16, V=16, seed=1)
    q, k, v, g, beta = (dev(d[n]) for n in ("q", "k", "v", "g", "beta"))
    o = torch.full((1, 8, 2, 16), 7.0, device="cuda:0")
    f = torch.full((1, 2, 16, 16), 7.0, device="cuda:0")
    L = binding.lib()
    P = lambda t: t.data_ptr()  # noqa: E731
    h = ctx.handle
    assert L.lrs_scan_delta_decay(h, P(q), P(k), P(v), None, P(beta), 1.0, None, P(o), P(f),
                                  1, 8, 2, 16, 16, None) == binding.LRS_E_INVAL        # g missing
    assert L.lrs_scan_delta_decay(h, P(q), P(k), P(v), P(g), P(beta), 1.0, None, P(o), P(f),
                                  1, 8, 2, 129, 16, None) == binding.LRS_E_UNSUPPORTED  # K > 128
    assert L.lrs_scan_delta_decay(h, P(q), P(k), P(v), P(g), P(beta), 1.0, None, P(o), P(o),
                                  1, 8, 2, 16, 16, None) == binding.LRS_E_INVAL        # outputs alias
    assert L.lrs_scan_delta_decay(h, P(q), P(k), P(v), P(g), P(beta), 1.0, None, P(g), P(f),
                                  1, 8, 2, 16, 16, None) == binding.LRS_E_INVAL        # output aliases g
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(f == 7.0)


def test_rwkv7_full_size_sampled(ctx):
    shape = inputs.RWKV7
    say(f"delta decay full size {shape}")
    d = inputs.rwkv7(**shape)
    o, fin = _gpu(ctx, d)
    for b, h in [(0, 0), (3, 11), (1, 5)]:
        sub = {n: (x[b:b + 1, :, h:h + 1] if n in SEQ else x) for n, x in d.items()}
        ro, rf = _ref(sub)
        eo = rel_heads(o[b:b + 1, :, h:h + 1], ro, "bthv")
        ef = rel_heads(fin[b:b + 1, h:h + 1], rf, "bhkv")
        say(f"   head ({b},{h}): rel err o={eo:.2e} s_final={ef:.2e}")
        assert eo <= TOL and ef <= TOL
    assert torch.isfinite(o).all() and torch.isfinite(fin).all()


def test_delta_decay_k128_full_size_all_heads(ctx):
    # the decayed delta rule at DeltaNet's full size (B=4, T=4096, H=8, K=V=128),
    # RWKV-7's decay law; on heads 0 and 5 of batch row 1 a stretch of steps
    # decays by 2 nats per step, so those chunks take the exact-exponential path
    shape = inputs.DELTA_DECAY_K128
    say(f"delta decay K=128 full size {shape}, all heads")
    d = inputs.rwkv7(**shape)
    g = d["g"].clone()
    g[1, 1000:1400, 0] = -2.0
    g[1, 3000:3100, 5, :64] = -2.0
    d["g"] = g
    o, fin = _gpu(ctx, d)
    ro, rf = _ref(d)
    eo, ef = rel_heads(o, ro, "bthv"), rel_heads(fin, rf, "bhkv")
    say(f"   worst slice rel err o={eo:.2e} s_final={ef:.2e}")
    assert eo <= TOL and ef <= TOL, (eo, ef)
