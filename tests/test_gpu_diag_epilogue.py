"""GPU parity of the decay-separable scan with its fused output epilogues
against the oracle's scan followed by the oracle's epilogue definitions,
through the C ABI: GLA's RMSNorm(o) * silu(g) [SunnyNet log §4.3], Mamba-2's
D x skip, and bf16 outputs.

Tolerance: fp32 outputs 2e-3 normwise per (batch, head) slice, as for the
scan itself.  A bf16 output adds its own rounding, at most 2^-8 of each value
(round to nearest with 8 significant bits), so bf16 outputs are held to
2e-3 + 2^-8 against the unrounded float64 oracle.  s_final is unaffected by
the epilogue and must still meet 2e-3.
"""
import pytest
import torch

import oracle
from linear_recurrence_scan_fma_amd import binding, inputs
from _helpers import dev, rel_heads, say

pytestmark = pytest.mark.gpu

TOL = 2e-3
TOL_BF16 = 2e-3 + 2.0 ** -8
F32, BF16 = binding.LRS_DTYPE_F32, binding.LRS_DTYPE_BF16


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = binding.Context(0)
    yield c
    c.close()


def _case(kind, B, T, H, K, V, seed, Hg=1):
    if kind == "skip":
        d = inputs.mamba2(B=B, T=T, H=H, K=K, V=V, seed=seed)
        d.update(inputs.skip_epilogue(H, seed=seed + 1))
        d["epilogue"] = binding.LRS_EPILOGUE_SKIP
    else:
        d = inputs.gla(B=B, T=T, H=H, K=K, V=V, seed=seed)
        d.update(inputs.norm_gate_epilogue(B, T, H, V, seed=seed + 1))
        d["epilogue"] = binding.LRS_EPILOGUE_NORM_GATE if kind == "norm_gate" else binding.LRS_EPILOGUE_NONE
    return d


def _gpu(ctx, d, out_dtype, s0=None):
    o, fin = binding.scan_diag_outer_epilogue(
        ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]), d["decay_mode"], dev(d["k_scale"]), d["scale"],
        dev(s0), d["epilogue"], dev(d.get("d_skip")), dev(d.get("gate")), dev(d.get("norm_weight")),
        d.get("eps", 0.0), out_dtype)
    torch.cuda.synchronize()
    return o, fin


def _ref(d, s0=None):
    o, fin = oracle.scan_diag_outer(d["q"], d["k"], d["v"], d["g"], d["decay_mode"], d["k_scale"], d["scale"],
                                    s0)
    if d["epilogue"] == binding.LRS_EPILOGUE_SKIP:
        o = oracle.epilogue_skip(o, d["d_skip"], d["v"])
    elif d["epilogue"] == binding.LRS_EPILOGUE_NORM_GATE:
        o = oracle.epilogue_norm_gate(o, d["gate"], d["norm_weight"], d["eps"])
    return o, fin


def _check(ctx, d, out_dtype, s0=None):
    o, fin = _gpu(ctx, d, out_dtype, s0)
    assert o.dtype == (torch.bfloat16 if out_dtype == BF16 else torch.float32)
    ro, rf = _ref(d, s0)
    eo, ef = rel_heads(o, ro, "bthv"), rel_heads(fin, rf, "bhkv")
    say(f"   rel err o={eo:.2e} s_final={ef:.2e}")
    assert eo <= (TOL_BF16 if out_dtype == BF16 else TOL) and ef <= TOL, (eo, ef)


SHAPES = [
    (2, 200, 4, 128, 64),     # Mamba-2 / GLA-like heads, ragged T
    (1, 150, 2, 128, 128),    # 8 waves per workgroup, whole row of 128 values
    (1, 130, 3, 100, 40),     # K, V not multiples of 8 (scalar loads and stores)
    (1, 1, 2, 64, 64),        # T = 1
]


@pytest.mark.parametrize("out_dtype", [F32, BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("kind", ["skip", "norm_gate", "none"])
def test_epilogue_parity(ctx, kind, shape, out_dtype):
    B, T, H, K, V = shape
    say(f"diag epilogue {kind} {shape} dtype={out_dtype}")
    d = _case(kind, B, T, H, K, V, seed=900 + T + K)
    _check(ctx, d, out_dtype, inputs.random_state((B, H, K, V), 25))


def test_epilogue_none_f32_equals_plain_call(ctx):
    d = _case("none", 1, 300, 2, 128, 128, seed=40)
    o1, f1 = _gpu(ctx, d, F32)
    o2, f2 = binding.scan_diag_outer(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]), 1, None, d["scale"])
    torch.cuda.synchronize()
    # a separately compiled variant: same arithmetic up to contraction choices
    assert rel_heads(o1, o2, "bthv") <= 1e-6 and rel_heads(f1, f2, "bhkv") <= 1e-6


def test_epilogue_norm_gate_eps_and_unit_weight(ctx):
    d = _case("norm_gate", 1, 200, 2, 128, 64, seed=41)
    d["norm_weight"] = None
    d["eps"] = 0.5
    _check(ctx, d, F32)


def test_epilogue_rejects_bad_arguments(ctx):
    d = _case("norm_gate", 1, 8, 2, 16, 256, seed=1)
    q, k, v, g, z = (dev(d[n]) for n in ("q", "k", "v", "g", "gate"))
    o = torch.full((1, 8, 2, 256), 7.0, device="cuda:0")
    f = torch.full((1, 2, 16, 256), 7.0, device="cuda:0")
    L = binding.lib()
    P = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    h = ctx.handle
    NG, SK = binding.LRS_EPILOGUE_NORM_GATE, binding.LRS_EPILOGUE_SKIP
    call = lambda epi, gate, dsk, dtype, V: L.lrs_scan_diag_outer_epilogue(  # noqa: E731
        h, P(q), P(k), P(v), P(g), 1, None, 1.0, None, epi, dsk, gate, None, 1e-6, dtype, P(o), P(f),
        1, 8, 2, 1, 16, V, None)
    assert call(NG, P(z), None, F32, 256) == binding.LRS_E_UNSUPPORTED   # the norm needs V <= 128
    assert call(NG, None, None, F32, 128) == binding.LRS_E_INVAL         # gate missing
    assert call(SK, None, None, F32, 128) == binding.LRS_E_INVAL         # D missing
    assert call(7, None, None, F32, 128) == binding.LRS_E_INVAL          # unknown epilogue
    assert call(0, None, None, 5, 128) == binding.LRS_E_INVAL            # unknown dtype
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(f == 7.0)


@pytest.mark.parametrize("which", ["gla_norm_gate", "mamba2_skip"])
def test_epilogue_full_size_sampled(ctx, which):
    if which == "gla_norm_gate":
        d = inputs.gla(**inputs.GLA)
        B, T, H, V = d["v"].shape
        d.update(inputs.norm_gate_epilogue(B, T, H, V))
        d["epilogue"] = binding.LRS_EPILOGUE_NORM_GATE
        heads = [(0, 0), (3, 3), (1, 2)]
    else:
        d = inputs.mamba2(**{k: v for k, v in inputs.MAMBA2.items() if k != "Hg"})
        B, T, H, V = d["v"].shape
        d.update(inputs.skip_epilogue(H))
        d["epilogue"] = binding.LRS_EPILOGUE_SKIP
        heads = [(0, 0), (7, 23), (3, 11)]
    say(f"diag epilogue full size {which}")
    o, fin = _gpu(ctx, d, BF16)
    for b, h in heads:
        sub = dict(d)
        for n in ("q", "k"):
            sub[n] = d[n][b:b + 1, :, (h if d[n].shape[2] > 1 else 0):][:, :, :1]
        for n in ("v", "g", "k_scale", "gate"):
            if d.get(n) is not None:
                sub[n] = d[n][b:b + 1, :, h:h + 1]
        if "d_skip" in d:
            sub["d_skip"] = d["d_skip"][h:h + 1]
        ro, rf = _ref(sub)
        eo = rel_heads(o[b:b + 1, :, h:h + 1], ro, "bthv")
        ef = rel_heads(fin[b:b + 1, h:h + 1], rf, "bhkv")
        say(f"   head ({b},{h}): rel err o={eo:.2e} s_final={ef:.2e}")
        assert eo <= TOL_BF16 and ef <= TOL
    assert torch.isfinite(o.float()).all() and torch.isfinite(fin).all()
