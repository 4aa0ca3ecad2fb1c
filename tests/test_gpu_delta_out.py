"""The delta rule (plain and with a per-key decay) with its output written as
bf16 or fp32 (lrs_scan_delta_out), against the sequential fp64 oracle.

Tolerances per (batch, head) slice, normwise: 2e-3 for the fp32 output and the
final state (bf16 inputs, fp32 state); 2e-3 + 2^-8 for a bf16 output (the
scan's tolerance plus the output's own round-to-nearest-even, 8 significant
bits).  The bf16 output is also the fp32 output rounded: within one bf16 step
of it element by element.
"""
import pytest
import torch

import oracle
from linear_recurrence_scan_fma_amd import binding, inputs
from _helpers import dev, rel_heads, say

pytestmark = pytest.mark.gpu

TOL = 2e-3
TOL_BF16 = 2e-3 + 2.0 ** -8


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = binding.Context(0)
    yield c
    c.close()


def _run(ctx, d, out_dtype, s0=None):
    g = dev(d["g"]) if "g" in d else None
    o, fin = binding.scan_delta_out(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["beta"]), g, d["scale"],
                                    dev(s0), out_dtype)
    torch.cuda.synchronize()
    return o, fin


def _ref(d, s0=None):
    if "g" in d:
        return oracle.scan_delta_decay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], s0)
    return oracle.scan_delta(d["q"], d["k"], d["v"], d["beta"], d["scale"], s0)


def _check_both(ctx, d, s0=None):
    ro, rf = _ref(d, s0)
    o32, f32 = _run(ctx, d, binding.LRS_DTYPE_F32, s0)
    o16, f16 = _run(ctx, d, binding.LRS_DTYPE_BF16, s0)
    assert o32.dtype == torch.float32 and o16.dtype == torch.bfloat16
    e32 = rel_heads(o32, ro, "bthv")
    e16 = rel_heads(o16.float(), ro, "bthv")
    ef = max(rel_heads(f32, rf, "bhkv"), rel_heads(f16, rf, "bhkv"))
    say(f"   rel err o fp32={e32:.2e} o bf16={e16:.2e} s_final={ef:.2e}")
    assert e32 <= TOL and ef <= TOL, (e32, ef)
    assert e16 <= TOL_BF16, e16
    # the bf16 output is the fp32 result rounded: within one bf16 step of it
    step = o32.abs() * 2.0 ** -7 + 1e-30
    assert torch.all((o16.float() - o32).abs() <= step)
    return o32, f32


@pytest.mark.parametrize("shape", [
    (2, 200, 3, 128, 128),   # DeltaNet head shape, ragged T
    (2, 150, 2, 64, 128),    # K = 64 != V = 128
    (1, 130, 2, 128, 40),    # ragged V tile
    (1, 77, 2, 36, 20),      # scalar loads
    (1, 1, 1, 128, 128),     # T = 1
], ids=lambda s: "x".join(map(str, s)))
def test_delta_out_plain(ctx, shape):
    B, T, H, K, V = shape
    say(f"delta out, plain {shape}")
    d = inputs.deltanet(B=B, T=T, H=H, K=K, V=V, seed=2400 + T + K)
    o32, f32 = _check_both(ctx, d, inputs.random_state((B, H, K, V), 2401))
    # the fp32 output of this entry point is the lrs_scan_delta call's
    o, fin = binding.scan_delta(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["beta"]), d["scale"],
                                dev(inputs.random_state((B, H, K, V), 2401)))
    torch.cuda.synchronize()
    assert torch.equal(o, o32) and torch.equal(fin, f32)


@pytest.mark.parametrize("shape", [
    (2, 200, 3, 64, 64),     # RWKV-7 head shape, ragged T
    (1, 100, 2, 48, 40),     # ragged K and V
    (1, 1, 1, 64, 64),       # T = 1
], ids=lambda s: "x".join(map(str, s)))
def test_delta_out_decay(ctx, shape):
    B, T, H, K, V = shape
    say(f"delta out, decayed {shape}")
    d = inputs.rwkv7(B=B, T=T, H=H, K=K, V=V, seed=2500 + T + K)
    _check_both(ctx, d, inputs.random_state((B, H, K, V), 2501))


def test_delta_out_rejects_bad_dtype_and_alignment(ctx):
    d = inputs.deltanet(B=1, T=8, H=2, K=16, V=16, seed=2)
    q, k, v, beta = (dev(d[n]) for n in ("q", "k", "v", "beta"))
    o = torch.empty((1, 8, 2, 17), device="cuda:0", dtype=torch.bfloat16)
    f = torch.empty((1, 2, 16, 16), device="cuda:0")
    L = binding.lib()
    P = lambda t: t.data_ptr()  # noqa: E731
    assert L.lrs_scan_delta_out(ctx.handle, P(q), P(k), P(v), None, P(beta), 1.0, None, 7, P(o), P(f),
                                1, 8, 2, 16, 16, None) == binding.LRS_E_INVAL          # unknown dtype
    assert L.lrs_scan_delta_out(ctx.handle, P(q), P(k), P(v), None, P(beta), 1.0, None, binding.LRS_DTYPE_F32,
                                P(o) + 2, P(f), 1, 8, 2, 16, 16, None) == binding.LRS_E_INVAL   # fp32 o, 2-byte aligned


FULL = {
    "deltanet_k128": lambda: inputs.deltanet(**inputs.DELTANET),
    "rwkv7": lambda: inputs.rwkv7(**inputs.RWKV7),
}


@pytest.mark.parametrize("name", list(FULL))
def test_delta_out_bf16_full_size_all_heads(ctx, name):
    say(f"delta out bf16, all heads, full size: {name}")
    d = FULL[name]()
    o16, fin = _run(ctx, d, binding.LRS_DTYPE_BF16)
    ro, rf = _ref(d)
    e16, ef = rel_heads(o16.float(), ro, "bthv"), rel_heads(fin, rf, "bhkv")
    say(f"   {name}: worst slice rel err o bf16={e16:.2e} s_final={ef:.2e}")
    assert e16 <= TOL_BF16 and ef <= TOL, (e16, ef)
