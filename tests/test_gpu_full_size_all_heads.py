"""Every output of every workload at its full size, in the launch
configuration the benchmark times, against the fp64 oracle run over the whole
workload on the host's threads.

Tolerances: normwise relative error <= 2e-3 per (batch, head) slice of o and
of s_final for the matrix-state scans (bf16 inputs, fp32 state); <= 1e-5 over
each whole output tensor for the fp32 elementwise scans.  Each case prints its
workload and its error before the assertion.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_recurrence_scan_fma_amd import binding, inputs
from _helpers import dev, rel_heads, say

pytestmark = pytest.mark.gpu

TOL = 2e-3
TOL_ELEM = 1e-5


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = binding.Context(0)
    yield c
    c.close()


def _check(name, o, fin, ro, rf):
    torch.cuda.synchronize()
    eo, ef = rel_heads(o, ro, "bthv"), rel_heads(fin, rf, "bhkv")
    say(f"   {name}: worst slice rel err o={eo:.2e} s_final={ef:.2e}")
    assert eo <= TOL and ef <= TOL, (eo, ef)


DIAG = {
    "mamba2": lambda: inputs.mamba2(**{k: v for k, v in inputs.MAMBA2.items() if k != "Hg"}),
    "gla": lambda: inputs.gla(**inputs.GLA),
    "hgrn2": lambda: inputs.hgrn2(**inputs.HGRN2),
    "assoc": lambda: inputs.assoc_memory(**inputs.ASSOC),
}


@pytest.mark.parametrize("name", list(DIAG))
def test_diag_outer_all_heads(ctx, name):
    say(f"all heads, full size: {name}")
    d = DIAG[name]()
    ksk = d.get("k_scale_key")
    if ksk is not None:
        o, fin = binding.scan_diag_outer_keyscale(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]),
                                                  dev(ksk), d["scale"])
    else:
        o, fin = binding.scan_diag_outer(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]),
                                         d["decay_mode"], dev(d["k_scale"]), d["scale"])
    ro, rf = oracle.scan_diag_outer(d["q"], d["k"], d["v"], d["g"], d["decay_mode"], d["k_scale"],
                                    d["scale"], k_scale_key=ksk)
    _check(name, o, fin, ro, rf)


DELTA = {
    "deltanet_k128": lambda: inputs.deltanet(**inputs.DELTANET),
    "deltanet_k64": lambda: inputs.deltanet(**inputs.DELTANET_K64),
    "rwkv7": lambda: inputs.rwkv7(**inputs.RWKV7),
}


@pytest.mark.parametrize("name", list(DELTA))
def test_delta_all_heads(ctx, name):
    say(f"all heads, full size: {name}")
    d = DELTA[name]()
    if "g" in d:
        o, fin = binding.scan_delta_decay(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]),
                                          dev(d["beta"]), d["scale"])
        ro, rf = oracle.scan_delta_decay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"])
    else:
        o, fin = binding.scan_delta(ctx, dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["beta"]), d["scale"])
        ro, rf = oracle.scan_delta(d["q"], d["k"], d["v"], d["beta"], d["scale"])
    _check(name, o, fin, ro, rf)


def _rel_rows(x, y):
    """Normwise relative error max|x - y| / max|y| of two [B, ...] tensors,
    accumulated one batch row at a time (bounded host memory)."""
    num, den = 0.0, 0.0
    for b in range(x.shape[0]):
        xb = x[b].detach().cpu().double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x[b], np.float64)
        yb = np.asarray(y[b], np.float64)
        if not np.all(np.isfinite(xb)):
            return float("inf")
        num = max(num, float(np.max(np.abs(xb - yb))))
        den = max(den, float(np.max(np.abs(yb))))
    return num / den if den > 0 else num


def test_gated_every_element(ctx):
    say("every element, full size: gated scan B=16 T=8192 N=2048")
    d = inputs.gated_large(**inputs.GATED_LARGE)
    a, u, s0 = d["a"], d["u"], d["s0"]
    binding.lrs_context_set_param(ctx, binding.LRS_PARAM_ELEM_SCHEDULE, binding.LRS_ELEM_SCHEDULE_AUTO)
    s, fin = binding.scan_elementwise(ctx, "gated", dev(a), dev(u), dev(s0))
    torch.cuda.synchronize()
    assert binding.lrs_context_check(ctx) == binding.LRS_OK
    rs, rf = oracle.scan_gated(a, u, s0)
    es, ef = _rel_rows(s, rs), _rel_rows(fin, rf)
    say(f"   gated: rel err s={es:.2e} s_final={ef:.2e}")
    assert es <= TOL_ELEM and ef <= TOL_ELEM, (es, ef)


def test_gated_backward_every_element(ctx):
    say("every element, full size: gated gradient pass B=16 T=8192 N=2048")
    cfg = inputs.GATED_LARGE
    B, T, N = cfg["B"], cfg["T"], cfg["N"]
    d = inputs.gated_large(**cfg)
    a, u, s0 = d["a"], d["u"], d["s0"]
    s = inputs.random_normal((B, T, N), 2001)
    ds = inputs.random_normal((B, T, N), 2002)
    dsf = inputs.random_state((B, N), 2003)
    binding.lrs_context_set_param(ctx, binding.LRS_PARAM_ELEM_SCHEDULE, binding.LRS_ELEM_SCHEDULE_AUTO)
    ad = dev(a)
    da, du = torch.empty_like(ad), torch.empty_like(ad)
    ds0 = torch.empty((B, N), device="cuda:0")
    binding.lrs_scan_gated_backward(ctx, ad, dev(u), dev(s0), dev(s), dev(ds), dev(dsf), da, du, ds0)
    torch.cuda.synchronize()
    assert binding.lrs_context_check(ctx) == binding.LRS_OK
    rda, rdu, rds0 = oracle.scan_gated_backward(a, u, s, ds, s0, dsf)
    ea, eu, e0 = _rel_rows(da, rda), _rel_rows(du, rdu), _rel_rows(ds0, rds0)
    say(f"   gated backward: rel err da={ea:.2e} du={eu:.2e} ds0={e0:.2e}")
    assert ea <= TOL_ELEM and eu <= TOL_ELEM and e0 <= TOL_ELEM, (ea, eu, e0)
