"""GPU parity with valid but not 16-byte-aligned tensors, against the fp64
oracle, through the C ABI.

The ABI asks for element alignment only (4 bytes for fp32, 2 for bf16);
16-byte alignment of every tensor selects the vector paths.  Here every
input and output is a view one element into a larger buffer (fp32 at 4 bytes
past a 16-byte boundary, bf16 at 2), at shapes whose sizes would otherwise
take the vector paths (N a multiple of 4, K and V multiples of 8), so each
scan family runs its scalar path on well-formed inputs.  The delta rule is
also run with aligned inputs and only its output (fp32 or bf16) misaligned:
its vector path stores four outputs per lane at once, so it must not be
chosen then.

Tolerances as for the aligned tests: normwise 1e-5 (elementwise), 2e-3 per
(batch, head) slice (matrix scans).
"""
import pytest
import torch

import oracle
from linear_recurrence_scan_fma_amd import binding, inputs
from _helpers import rel, rel_heads, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = binding.Context(0)
    yield c
    c.close()


def _off(t, shape=None, dtype=None):
    """A contiguous device view one element into a fresh buffer, holding t
    (or uninitialised, for outputs: t None, shape and dtype given)."""
    shape = tuple(t.shape) if t is not None else tuple(shape)
    dtype = t.dtype if t is not None else dtype
    n = 1
    for x in shape:
        n *= x
    buf = torch.empty(n + 1, dtype=dtype, device="cuda:0")
    view = buf[1:].view(shape)
    if t is not None:
        view.copy_(t.to("cuda:0"))
    assert view.data_ptr() % 16 != 0
    return view


@pytest.mark.parametrize("kind", ["fma", "gated"])
def test_elementwise_misaligned(ctx, kind):
    B, T, N = 2, 1000, 256
    say(f"elem {kind} misaligned B={B} T={T} N={N}")
    d = inputs.elementwise_small(B, T, N, seed=4201)
    x = d["b"] if kind == "fma" else d["u"]
    s0 = inputs.random_state((B, N), 4202)
    s = _off(None, (B, T, N), torch.float32)
    fin = _off(None, (B, N), torch.float32)
    fn = binding.lrs_scan_fma if kind == "fma" else binding.lrs_scan_gated
    fn(ctx, _off(d["a"]), _off(x), _off(s0), s, fin)
    torch.cuda.synchronize()
    assert binding.lrs_context_check(ctx) == binding.LRS_OK
    rs, rf = (oracle.scan_fma if kind == "fma" else oracle.scan_gated)(d["a"], x, s0)
    err = max(rel(s, rs), rel(fin, rf))
    say(f"   rel err {err:.2e}")
    assert err <= 1e-5, err


@pytest.mark.parametrize("kind", ["fma", "gated"])
def test_step_misaligned(ctx, kind):
    B, N = 16, 2048
    say(f"step {kind} misaligned B={B} N={N}")
    d = inputs.elementwise_small(B, 1, N, seed=4208)
    x = d["b"] if kind == "fma" else d["u"]
    s0 = inputs.random_state((B, N), 4209)
    s = _off(s0)
    (binding.lrs_step_fma if kind == "fma" else binding.lrs_step_gated)(ctx, _off(d["a"][:, 0]), _off(x[:, 0]), s)
    torch.cuda.synchronize()
    # one step is the one-step scan
    rs, _ = (oracle.scan_fma if kind == "fma" else oracle.scan_gated)(d["a"], x, s0)
    err = rel(s, rs[:, 0])
    say(f"   rel err {err:.2e}")
    assert err <= 1e-5, err


@pytest.mark.parametrize("decay", [False, True], ids=["plain", "decayed"])
def test_delta_misaligned(ctx, decay):
    B, T, H, K, V = 1, 200, 2, 128 if not decay else 64, 128 if not decay else 64
    say(f"delta {'decayed' if decay else 'plain'} misaligned B={B} T={T} H={H} K={K} V={V}")
    d = inputs.rwkv7(B=B, T=T, H=H, K=K, V=V, seed=4203) if decay else \
        inputs.deltanet(B=B, T=T, H=H, K=K, V=V, seed=4203)
    s0 = inputs.random_state((B, H, K, V), 4204, std=0.1)
    o = _off(None, (B, T, H, V), torch.float32)
    fin = _off(None, (B, H, K, V), torch.float32)
    q, k, v, beta = (_off(d[n]) for n in ("q", "k", "v", "beta"))
    if decay:
        binding.lrs_scan_delta_decay(ctx, q, k, v, _off(d["g"]), beta, d["scale"], _off(s0), o, fin)
    else:
        binding.lrs_scan_delta(ctx, q, k, v, beta, d["scale"], _off(s0), o, fin)
    torch.cuda.synchronize()
    if decay:
        ro, rf = oracle.scan_delta_decay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], s0)
    else:
        ro, rf = oracle.scan_delta(d["q"], d["k"], d["v"], d["beta"], d["scale"], s0)
    eo, ef = rel_heads(o, ro, "bthv"), rel_heads(fin, rf, "bhkv")
    say(f"   rel err o={eo:.2e} s_final={ef:.2e}")
    assert eo <= 2e-3 and ef <= 2e-3, (eo, ef)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("decay", [False, True], ids=["plain", "decayed"])
def test_delta_aligned_inputs_misaligned_output(ctx, decay, out):
    # only the output is off a 16-byte boundary: the call must not take the
    # vector path, whose lanes store four outputs at once
    B, T, H = 1, 200, 2
    K = V = 64 if decay else 128
    say(f"delta {'decayed' if decay else 'plain'} aligned inputs, misaligned {out} output")
    d = inputs.rwkv7(B=B, T=T, H=H, K=K, V=V, seed=4207) if decay else \
        inputs.deltanet(B=B, T=T, H=H, K=K, V=V, seed=4207)
    dd = {n: d[n].to("cuda:0") for n in ("q", "k", "v", "beta") + (("g",) if decay else ())}
    odt = torch.float32 if out == "f32" else torch.bfloat16
    o = _off(None, (B, T, H, V), odt)
    fin = torch.empty((B, H, K, V), dtype=torch.float32, device="cuda:0")
    binding.lrs_scan_delta_out(ctx, dd["q"], dd["k"], dd["v"], dd.get("g"), dd["beta"], d["scale"], None,
                               binding.LRS_DTYPE_F32 if out == "f32" else binding.LRS_DTYPE_BF16, o, fin)
    torch.cuda.synchronize()
    if decay:
        ro, rf = oracle.scan_delta_decay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], None)
    else:
        ro, rf = oracle.scan_delta(d["q"], d["k"], d["v"], d["beta"], d["scale"], None)
    eo, ef = rel_heads(o, ro, "bthv"), rel_heads(fin, rf, "bhkv")
    say(f"   rel err o={eo:.2e} s_final={ef:.2e}")
    # a bf16 output adds its own rounding, 2^-8 relative
    assert eo <= (2e-3 if out == "f32" else 2e-3 + 2.0 ** -8) and ef <= 2e-3, (eo, ef)


@pytest.mark.parametrize("family", ["mamba2", "gla"])
def test_diag_outer_misaligned(ctx, family):
    say(f"diag {family} misaligned")
    if family == "mamba2":
        d = inputs.mamba2(B=1, T=200, H=3, K=128, V=64, seed=4205)
    else:
        d = inputs.gla(B=1, T=200, H=2, K=128, V=128, seed=4205)
    B, T, H, V = d["v"].shape
    K = d["q"].shape[3]
    s0 = inputs.random_state((B, H, K, V), 4206, std=0.1)
    o = _off(None, (B, T, H, V), torch.float32)
    fin = _off(None, (B, H, K, V), torch.float32)
    ks = _off(d["k_scale"]) if d["k_scale"] is not None else None
    binding.lrs_scan_diag_outer(ctx, _off(d["q"]), _off(d["k"]), _off(d["v"]), _off(d["g"]), d["decay_mode"], ks,
                                d["scale"], _off(s0), o, fin)
    torch.cuda.synchronize()
    ro, rf = oracle.scan_diag_outer(d["q"], d["k"], d["v"], d["g"], d["decay_mode"], d["k_scale"], d["scale"], s0)
    eo, ef = rel_heads(o, ro, "bthv"), rel_heads(fin, rf, "bhkv")
    say(f"   rel err o={eo:.2e} s_final={ef:.2e}")
    assert eo <= 2e-3 and ef <= 2e-3, (eo, ef)
