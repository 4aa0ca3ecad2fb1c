"""GPU parity of the decay-separable scan with a per-key injection scale (the
matrix associative memory [vs llama.cpp §8]: S_t = p (.) S_{t-1} + (1 - p) (.)
(v_t (x) k_t) with p on the key axis, as g = log p and kappa = 1 - p) and of the
HGRN2-shaped scan (GLA's recurrence with the key tied to the forget gate,
[vs llama.cpp §4]) against the sequential fp64 oracle, through the C ABI.

Tolerance: normwise relative error <= 2e-3 per (batch, head) slice of o and of
s_final, as for the other matrix scans.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_recurrence_scan_fma_amd import binding, inputs
from _helpers import dev, rel_heads, say

pytestmark = pytest.mark.gpu

TOL = 2e-3
SEQ = ("q", "k", "v", "g", "k_scale_key")


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = binding.Context(0)
    yield c
    c.close()


class _Segments:
    """Sets LRS_PARAM_DIAG_SEGMENTS for a block and restores the default."""

    def __init__(self, ctx, n):
        self.ctx, self.n = ctx, n

    def __enter__(self):
        binding.lrs_context_set_param(self.ctx, binding.LRS_PARAM_DIAG_SEGMENTS, self.n)

    def __exit__(self, *exc):
        binding.lrs_context_set_param(self.ctx, binding.LRS_PARAM_DIAG_SEGMENTS, 0)


def _gpu(ctx, d, s0=None):
    o, fin = binding.scan_diag_outer_keyscale(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]),
                                              dev(d["k_scale_key"]), d["scale"], dev(s0))
    torch.cuda.synchronize()
    return o, fin


def _ref(d, s0=None):
    return oracle.scan_diag_outer(d["q"], d["k"], d["v"], d["g"], 1, None, d["scale"], s0,
                                  k_scale_key=d["k_scale_key"])


def _check(ctx, d, s0=None):
    o, fin = _gpu(ctx, d, s0)
    ro, rf = _ref(d, s0)
    eo, ef = rel_heads(o, ro, "bthv"), rel_heads(fin, rf, "bhkv")
    say(f"   rel err o={eo:.2e} s_final={ef:.2e}")
    assert eo <= TOL and ef <= TOL, (eo, ef)


def _assoc(B, T, H, K, V, seed, Hg=None):
    d = inputs.assoc_memory(B=B, T=T, H=H, K=K, V=V, seed=seed)
    if Hg is not None and Hg != H:   # grouped q/k: one q/k row per group
        d["q"], d["k"] = d["q"][:, :, :Hg].contiguous(), d["k"][:, :, :Hg].contiguous()
    return d


@pytest.mark.parametrize("shape", [
    (2, 200, 4, 4, 64, 64),     # associative-memory head shape, ragged T
    (1, 64, 2, 2, 64, 64),      # one chunk
    (1, 150, 2, 1, 128, 128),   # K = V = 128: 8 waves per workgroup, one q/k group
    (2, 300, 4, 2, 128, 64),    # two groups
    (1, 130, 3, 3, 100, 37),    # K, V not multiples of 8 (scalar loads)
    (1, 1, 1, 1, 64, 64),       # T = 1
    (2, 70, 2, 2, 1, 1),        # K = V = 1
], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_s0", [False, True])
def test_keyscale_parity(ctx, shape, with_s0):
    B, T, H, Hg, K, V = shape
    say(f"diag keyscale {shape} s0={with_s0}")
    d = _assoc(B, T, H, K, V, seed=800 + T + K, Hg=Hg)
    s0 = inputs.random_state((B, H, K, V), 21) if with_s0 else None
    _check(ctx, d, s0)


@pytest.mark.parametrize("segments", [1, 3, 7])
def test_keyscale_time_segments(ctx, segments):
    B, T, H, K, V = 1, 900, 2, 64, 64
    d = _assoc(B, T, H, K, V, seed=31)
    with _Segments(ctx, segments):
        _check(ctx, d, inputs.random_state((B, H, K, V), 22))


@pytest.mark.parametrize("segments", [1, 3])
def test_keyscale_strong_decay_exact_path(ctx, segments):
    # p = 0.05: 3 nats per step, past the factorised path's range in every chunk
    B, T, H, K, V = 1, 260, 2, 128, 64
    d = _assoc(B, T, H, K, V, seed=32)
    p = torch.full_like(d["g"], 0.05)
    p[:, ::3] = 0.9
    d["g"] = torch.log(p)
    d["k_scale_key"] = 1.0 - p
    with _Segments(ctx, segments):
        _check(ctx, d, inputs.random_state((B, H, K, V), 23))


def test_keyscale_equal_on_keys_is_the_per_head_scale(ctx):
    B, T, H, K, V = 1, 200, 2, 128, 128
    d = inputs.gla(B=B, T=T, H=H, K=K, V=V, seed=33)
    ks = torch.from_numpy(np.random.default_rng(34).uniform(0.2, 2.0, (B, T, H)).astype(np.float32))
    o1, f1 = binding.scan_diag_outer(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]), 1, dev(ks),
                                     d["scale"])
    o2, f2 = binding.scan_diag_outer_keyscale(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]),
                                              dev(ks[..., None].expand(B, T, H, K).contiguous()), d["scale"])
    torch.cuda.synchronize()
    assert rel_heads(o2, o1, "bthv") <= 1e-5 and rel_heads(f2, f1, "bhkv") <= 1e-5


def test_keyscale_continuation(ctx):
    B, T, H, K, V = 1, 260, 2, 64, 64
    d = _assoc(B, T, H, K, V, seed=35)
    s0 = inputs.random_state((B, H, K, V), 24)
    o_full, f_full = _gpu(ctx, d, s0)
    for t1 in (1, 64, 130):
        first = {n: (x[:, :t1] if n in SEQ else x) for n, x in d.items()}
        second = {n: (x[:, t1:] if n in SEQ else x) for n, x in d.items()}
        o1, f1 = _gpu(ctx, first, s0)
        o2, f2 = _gpu(ctx, second, f1.cpu())
        assert rel_heads(torch.cat([o1, o2], 1), o_full, "bthv") <= 1e-4
        assert rel_heads(f2, f_full, "bhkv") <= 1e-4


def test_keyscale_rejects_bad_arguments(ctx):
    d = _assoc(1, 8, 2, 16, 16, seed=1)
    q, k, v, g, ks = (dev(d[n]) for n in ("q", "k", "v", "g", "k_scale_key"))
    o = torch.full((1, 8, 2, 16), 7.0, device="cuda:0")
    f = torch.full((1, 2, 16, 16), 7.0, device="cuda:0")
    L = binding.lib()
    P = lambda t: t.data_ptr()  # noqa: E731
    h = ctx.handle
    assert L.lrs_scan_diag_outer_keyscale(h, P(q), P(k), P(v), P(g), None, 1.0, None, P(o), P(f),
                                          1, 8, 2, 2, 16, 16, None) == binding.LRS_E_INVAL   # kappa missing
    assert L.lrs_scan_diag_outer_keyscale(h, P(q), P(k), P(v), P(g), P(ks), 1.0, None, P(o), P(f),
                                          1, 8, 2, 2, 129, 16, None) == binding.LRS_E_UNSUPPORTED
    assert L.lrs_scan_diag_outer_keyscale(h, P(q), P(k), P(v), P(g), P(ks), 1.0, None, P(ks), P(f),
                                          1, 8, 2, 2, 16, 16, None) == binding.LRS_E_INVAL   # o aliases kappa
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(f == 7.0)


def test_assoc_memory_full_size_sampled(ctx):
    shape = inputs.ASSOC
    say(f"assoc memory full size {shape}")
    d = inputs.assoc_memory(**shape)
    o, fin = _gpu(ctx, d)
    for b, h in [(0, 0), (3, 7), (2, 3)]:
        sub = {n: (x[b:b + 1, :, h:h + 1] if n in SEQ else x) for n, x in d.items()}
        ro, rf = _ref(sub)
        eo = rel_heads(o[b:b + 1, :, h:h + 1], ro, "bthv")
        ef = rel_heads(fin[b:b + 1, h:h + 1], rf, "bhkv")
        say(f"   head ({b},{h}): rel err o={eo:.2e} s_final={ef:.2e}")
        assert eo <= TOL and ef <= TOL
    assert torch.isfinite(o).all() and torch.isfinite(fin).all()


# ---- HGRN2 shape: GLA's call with k = 1 - f ----------------------------------
def _gla_call(ctx, d):
    o, fin = binding.scan_diag_outer(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]), 1, None,
                                     d["scale"])
    torch.cuda.synchronize()
    return o, fin


def test_hgrn2_small_parity(ctx):
    d = inputs.hgrn2(B=2, T=300, H=3, K=128, V=128, seed=36)
    o, fin = _gla_call(ctx, d)
    ro, rf = oracle.scan_diag_outer(d["q"], d["k"], d["v"], d["g"], 1, None, d["scale"])
    assert rel_heads(o, ro, "bthv") <= TOL and rel_heads(fin, rf, "bhkv") <= TOL


def test_hgrn2_full_size_sampled(ctx):
    shape = inputs.HGRN2
    say(f"hgrn2 full size {shape}")
    d = inputs.hgrn2(**shape)
    o, fin = _gla_call(ctx, d)
    for b, h in [(0, 0), (3, 15), (1, 8)]:
        sub = {n: (x[b:b + 1, :, h:h + 1] if n in ("q", "k", "v", "g") else x) for n, x in d.items()}
        ro, rf = oracle.scan_diag_outer(sub["q"], sub["k"], sub["v"], sub["g"], 1, None, d["scale"])
        eo = rel_heads(o[b:b + 1, :, h:h + 1], ro, "bthv")
        ef = rel_heads(fin[b:b + 1, h:h + 1], rf, "bhkv")
        say(f"   head ({b},{h}): rel err o={eo:.2e} s_final={ef:.2e}")
        assert eo <= TOL and ef <= TOL
    assert torch.isfinite(o).all() and torch.isfinite(fin).all()
