"""GPU parity on long sequences (T = 65,536 steps for the matrix scans, 2^20
for the elementwise scan) against the sequential fp64 oracle, through the C
ABI.  One (batch, head) slice walks 1,024 chunks, so these cases cover the
paths a long single-stream call takes: many time segments (decay-separable
scans and the delta rule at batch 1 split the time axis by themselves), a
single segment walking every chunk (forced), and thousands of look-back tiles
in a row.  Error must not build up along the sequence: besides the normwise
error over the whole slice, the last 4,096 steps are checked on their own.

The decaying families take their decay scaled down (log-decay times 1e-3,
GLA's times 1e-2): at the workloads' own rates the state a segment inherits
decays below fp32 resolution within a few hundred steps, so the segmented
and the one-pass calls return identical bits and the carry between segments
would go untested.  Weakened, the carry stays significant across segments
(the delta rule without decay carries its state in full).

Tolerances as in the per-scan tests: 2e-3 normwise per (batch, head) slice
for the matrix scans, 1e-5 for the elementwise scan.
"""
import pytest
import torch

import oracle
from linear_recurrence_scan_fma_amd import binding, inputs
from _helpers import dev, rel, rel_heads, say

pytestmark = pytest.mark.gpu

T_LONG = 65536
TAIL = 4096


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = binding.Context(0)
    yield c
    for prm in (binding.LRS_PARAM_DELTA_SEGMENTS, binding.LRS_PARAM_DIAG_SEGMENTS,
                binding.LRS_PARAM_ELEM_SCHEDULE):
        binding.lrs_context_set_param(c, prm, 0)
    c.close()


def _check(name, o, fin, ro, rf, tol):
    eo, ef = rel_heads(o, ro, "bthv"), rel_heads(fin, rf, "bhkv")
    et = rel_heads(o[:, -TAIL:], ro[:, -TAIL:], "bthv")
    say(f"   {name}: rel err o={eo:.2e} last {TAIL} steps={et:.2e} s_final={ef:.2e}")
    assert eo <= tol and et <= tol and ef <= tol, (eo, et, ef)


@pytest.mark.parametrize("segments", [0, 1], ids=["auto", "one_pass"])
@pytest.mark.parametrize("family", ["deltanet", "rwkv7"])
def test_delta_long(ctx, family, segments):
    K = V = 128 if family == "deltanet" else 64
    say(f"delta {family} B=1 T={T_LONG} H=1 K={K} V={V} segments={segments}")
    binding.lrs_context_set_param(ctx, binding.LRS_PARAM_DELTA_SEGMENTS, segments)
    if family == "deltanet":
        d = inputs.deltanet(B=1, T=T_LONG, H=1, K=K, V=V, seed=901)
        o, fin = binding.scan_delta(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["beta"]), d["scale"], None)
        torch.cuda.synchronize()
        ro, rf = oracle.scan_delta(d["q"], d["k"], d["v"], d["beta"], d["scale"], None)
    else:
        d = inputs.rwkv7(B=1, T=T_LONG, H=1, K=K, V=V, seed=902)
        d["g"] = d["g"] * 1e-3
        o, fin = binding.scan_delta_decay(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]), dev(d["beta"]),
                                          d["scale"], None)
        torch.cuda.synchronize()
        ro, rf = oracle.scan_delta_decay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], None)
    binding.lrs_context_set_param(ctx, binding.LRS_PARAM_DELTA_SEGMENTS, 0)
    _check(family, o, fin, ro, rf, 2e-3)


@pytest.mark.parametrize("segments", [0, 1], ids=["auto", "one_pass"])
@pytest.mark.parametrize("family", ["gla", "mamba2"])
def test_diag_outer_long(ctx, family, segments):
    say(f"diag {family} B=1 T={T_LONG} segments={segments}")
    binding.lrs_context_set_param(ctx, binding.LRS_PARAM_DIAG_SEGMENTS, segments)
    if family == "gla":
        d = inputs.gla(B=1, T=T_LONG, H=1, K=128, V=128, seed=903)
        d["g"] = d["g"] * 1e-2
    else:
        d = inputs.mamba2(B=1, T=T_LONG, H=2, K=128, V=64, seed=904)
        d["g"] = d["g"] * 1e-3
    o, fin = binding.scan_diag_outer(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]), d["decay_mode"],
                                     dev(d["k_scale"]), d["scale"], None)
    torch.cuda.synchronize()
    binding.lrs_context_set_param(ctx, binding.LRS_PARAM_DIAG_SEGMENTS, 0)
    ro, rf = oracle.scan_diag_outer(d["q"], d["k"], d["v"], d["g"], d["decay_mode"], d["k_scale"], d["scale"], None)
    _check(family, o, fin, ro, rf, 2e-3)


@pytest.mark.parametrize("schedule", [binding.LRS_ELEM_SCHEDULE_STREAM, binding.LRS_ELEM_SCHEDULE_LOOKBACK],
                         ids=["stream", "lookback"])
def test_gated_long(ctx, schedule):
    B, T, N = 1, 1 << 20, 64
    say(f"elem gated B={B} T={T} N={N} schedule={schedule}")
    d = inputs.gated_large(B=B, T=T, N=N, seed=905)
    binding.lrs_context_set_param(ctx, binding.LRS_PARAM_ELEM_SCHEDULE, schedule)
    s, fin = binding.scan_elementwise(ctx, "gated", dev(d["a"]), dev(d["u"]), dev(d["s0"]))
    torch.cuda.synchronize()
    binding.lrs_context_set_param(ctx, binding.LRS_PARAM_ELEM_SCHEDULE, 0)
    assert binding.lrs_context_check(ctx) == binding.LRS_OK
    rs, rf = oracle.scan_gated(d["a"], d["u"], d["s0"])
    es, et, ef = rel(s, rs), rel(s[:, -TAIL:], rs[:, -TAIL:]), rel(fin, rf)
    say(f"   rel err s={es:.2e} last {TAIL} steps={et:.2e} s_final={ef:.2e}")
    assert es <= 1e-5 and et <= 1e-5 and ef <= 1e-5, (es, et, ef)
    assert torch.equal(fin, s[:, -1])
