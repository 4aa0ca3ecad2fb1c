"""GPU parity of the delta rule run in time segments (LRS_PARAM_DELTA_SEGMENTS)
against the sequential fp64 oracle, through the C ABI.

A segmented call computes each segment's transition S_out = A_s S_in + B_s
(A_s from identity columns run through the update with zero values), chains
the segments' entering states, and runs every segment's outputs at once: the
same recurrence [SunnyNet log §4.2, §5.1] regrouped over the time axis.  The
cases force segment counts on ragged shapes (vector and scalar paths, with an
initial state, K != V, the decayed form, a bf16 output) and check the
automatic choice at batch 1, where it splits the time axis.

Tolerance: normwise relative error <= 2e-3 per (batch, head) slice of o and of
s_final, as for the unsegmented calls (bf16 output: 2e-3 + 2^-8).
"""
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
    binding.lrs_context_set_param(c, binding.LRS_PARAM_DELTA_SEGMENTS, 0)
    c.close()


def _run(ctx, d, s0, nseg, decay, out_dtype=binding.LRS_DTYPE_F32):
    binding.lrs_context_set_param(ctx, binding.LRS_PARAM_DELTA_SEGMENTS, nseg)
    q, k, v, beta = (dev(d[n]) for n in ("q", "k", "v", "beta"))
    B, T, H, K = q.shape
    V = v.shape[3]
    dt = torch.bfloat16 if out_dtype == binding.LRS_DTYPE_BF16 else torch.float32
    o = torch.empty((B, T, H, V), dtype=dt, device=q.device)
    fin = torch.empty((B, H, K, V), dtype=torch.float32, device=q.device)
    binding.lrs_scan_delta_out(ctx, q, k, v, dev(d["g"]) if decay else None, beta, d["scale"], dev(s0),
                               out_dtype, o, fin)
    torch.cuda.synchronize()
    return o.float(), fin


def _ref(d, s0, decay):
    if decay:
        return oracle.scan_delta_decay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], s0)
    return oracle.scan_delta(d["q"], d["k"], d["v"], d["beta"], d["scale"], s0)


@pytest.mark.parametrize("nseg", [2, 3, 5])
@pytest.mark.parametrize("shape,decay", [
    ((1, 1000, 2, 128, 128), False),   # DeltaNet head, ragged T
    ((2, 700, 1, 64, 128), False),     # K = 64 != V = 128
    ((1, 900, 2, 100, 40), False),     # K, V not multiples of 8 (scalar loads), ragged V tile
    ((1, 800, 2, 64, 64), True),       # RWKV-7 head, decayed
    ((1, 650, 1, 128, 128), True),     # decayed at K = 128
], ids=lambda x: "x".join(map(str, x)) if isinstance(x, tuple) else str(x))
def test_segments_parity(ctx, shape, decay, nseg):
    B, T, H, K, V = shape
    say(f"delta segments {shape} decay={decay} nseg={nseg}")
    d = (inputs.rwkv7 if decay else inputs.deltanet)(B=B, T=T, H=H, K=K, V=V, seed=500 + T + K + nseg)
    s0 = inputs.random_state((B, H, K, V), 21)
    o, fin = _run(ctx, d, s0, nseg, decay)
    ro, rf = _ref(d, s0, decay)
    eo, ef = rel_heads(o, ro, "bthv"), rel_heads(fin, rf, "bhkv")
    say(f"   rel err o={eo:.2e} s_final={ef:.2e}")
    assert eo <= TOL and ef <= TOL, (eo, ef)


def test_segments_bf16_output(ctx):
    d = inputs.deltanet(B=1, T=1100, H=2, K=128, V=128, seed=531)
    o, fin = _run(ctx, d, None, 4, False, binding.LRS_DTYPE_BF16)
    ro, rf = _ref(d, None, False)
    assert rel_heads(o, ro, "bthv") <= TOL + 2.0 ** -8 and rel_heads(fin, rf, "bhkv") <= TOL


def test_segments_agree_with_one_pass(ctx):
    # the segmented and the one-pass call agree with each other as with the oracle
    d = inputs.deltanet(B=1, T=2048, H=4, K=128, V=128, seed=532)
    o1, f1 = _run(ctx, d, None, 1, False)
    o3, f3 = _run(ctx, d, None, 3, False)
    assert rel_heads(o3, o1, "bthv") <= TOL and rel_heads(f3, f1, "bhkv") <= TOL


@pytest.mark.parametrize("decay", [False, True])
def test_auto_segments_batch_one(ctx, decay):
    # batch 1: the (head, V-tile) workgroups fill a quarter of the chip, so the
    # automatic choice splits the time axis
    shape = dict(B=1, T=4096, H=8, K=128, V=128)
    say(f"delta auto segments {shape} decay={decay}")
    d = (inputs.rwkv7 if decay else inputs.deltanet)(**shape, seed=540 + int(decay))
    o, fin = _run(ctx, d, None, 0, decay)
    ro, rf = _ref(d, None, decay)
    eo, ef = rel_heads(o, ro, "bthv"), rel_heads(fin, rf, "bhkv")
    say(f"   rel err o={eo:.2e} s_final={ef:.2e}")
    assert eo <= TOL and ef <= TOL, (eo, ef)
