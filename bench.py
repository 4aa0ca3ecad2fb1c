"""Throughput of the scan library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-rows] [--no-cpu]

Headline (the JSON line's `value`): the gated elementwise scan
s_t = a_t s_{t-1} + (1 - a_t) u_t on B=16, T=8192, N=2048 fp32 with an fp32
initial state, inputs resident in HBM.  One step = one lrs_scan_gated call over
that batch.  `value` is algorithmic GB/s (inputs read once, outputs written
once) over the wall-clock of K steps; `roofline.achieved` uses the average
kernel duration from HIP events recorded on the launch stream, and
`roofline.frac_of_copy` relates it to a 1 GiB device copy measured in the
same run.

`rows` reports the other scans at their workload shapes, each measured in a
process of its own (`python bench.py --row NAME`), with per-launch event
timing after a 512 MB read that evicts the call's inputs from the 256 MB
last-level cache, its own roofline figure, parity against the oracle, and the
oracle timed on this host (all granted threads on the whole workload, and one
thread on a stated sample).  Small calls report host and GPU time separately.

`cpu_baseline` is the sequential CPU oracle (fp64) timed on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "linear_recurrence_scan_fma_amd", "csrc")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha(name):
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def profile_record(kernel_key, source_file):
    """The rocprofv3 record of a kernel in profiles/traffic.json, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec or rec.get("source_sha") != source_sha(source_file):
        return None
    return rec


def measured_traffic(kernel_key, source_file):
    """HBM bytes per launch measured by rocprofv3 counters (current source only)."""
    rec = profile_record(kernel_key, source_file)
    return None if rec is None else rec.get("bytes_per_launch")


def measured_kernel_us(kernel_key, source_file):
    """Average kernel duration from the rocprofv3 kernel trace (current source only)."""
    rec = profile_record(kernel_key, source_file)
    return None if rec is None or "avg_ns" not in rec else round(rec["avg_ns"] / 1e3, 3)


def measured_mfma_util(kernel_keys, source_file):
    """Matrix-core busy fraction of SIMD cycles over a call's kernels (busy
    cycles summed over kernels / active cycles x SIMDs), from counters taken
    on the current source; else None."""
    recs = [profile_record(k, source_file) for k in kernel_keys]
    if any(r is None or "mfma_busy_cycles" not in r for r in recs):
        return None
    busy = sum(r["mfma_busy_cycles"] for r in recs)
    active = sum(r["gui_active_cycles_sum_xcd"] for r in recs)
    return round(busy * 8 / (active * 1024), 4) if active else None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def elem_bytes(B, T, N, with_s0=True):
    return 12 * B * T * N + 4 * B * N + (4 * B * N if with_s0 else 0)


def digests(d, names):
    from linear_recurrence_scan_fma_amd import inputs

    return {n: inputs.digest(d[n]) for n in names if d.get(n) is not None}


def time_steps(fn, steps, warmup):
    """Runs fn warmup times, then times `steps` calls: wall clock with a
    synchronize on both sides, and HIP events on the current stream."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps


def time_launches(fn, reps, warmup, flush):
    """Median and min of per-launch HIP-event times on the current stream, with
    the 256 MB last-level cache emptied of the call's data before each launch.

    The eviction reads a 512 MB buffer (a reduction), so the cache is left
    holding clean lines only: a write-based flush would leave up to 256 MB of
    its own dirty lines, whose write-back the timed call would then pay for.
    The reduction is queued ahead of the timed call without a host wait, as the
    call would be queued behind other work in a pipeline."""
    import torch

    stream = torch.cuda.current_stream()
    ts = []
    for i in range(warmup + reps):
        flush.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= warmup:
            ts.append(e0.elapsed_time(e1))
    ts.sort()
    return ts[len(ts) // 2], ts[0]


def copy_gbs(dev):
    """Device-to-device bandwidth of a 1 GiB tensor copy (2 GiB moved), the
    best of 10 event-timed copies."""
    import torch

    src = torch.ones(1 << 28, device=dev)
    dst = torch.empty_like(src)
    best = None
    for i in range(12):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
    del src, dst
    return 2 * (1 << 30) / (best * 1e-3) / 1e9


def roofline(nbytes, ms, copy=None):
    achieved = nbytes / (ms * 1e-3) / 1e9
    r = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(achieved / HBM_PEAK_GBS, 4), "bytes_per_call": nbytes}
    if copy:
        r["frac_of_copy"] = round(achieved / copy, 4)
    return r


def oracle_cpu(fn_all, fn_one, units, unit, sample_all, sample_one, units_one):
    """Times the oracle with every granted thread (fn_all) and on one thread
    (fn_one, a stated sample); returns the cpu_baseline object."""
    import oracle

    nth = oracle.default_threads()
    t0 = time.perf_counter()
    res = fn_all(nth)
    dt = time.perf_counter() - t0
    t0 = time.perf_counter()
    fn_one(1)
    dt1 = time.perf_counter() - t0
    return res, {"value": round(units / dt, 3), "unit": unit, "cores": nth, "kind": "oracle",
                 "sample": sample_all, "seconds": round(dt, 3), "cpu_model": cpu_model(),
                 "single_thread": {"value": round(units_one / dt1, 3), "unit": unit, "cores": 1,
                                   "sample": sample_one, "seconds": round(dt1, 3)}}


# ---------------------------------------------------------------------------
# rows (each runs in its own process)
# ---------------------------------------------------------------------------
STEP_SMALL = (16, 2048)        # one decode step of the gated workload's state
STEP_LARGE = (16, 4194304)     # 2^26 channels: 1 GiB moved per step


def elem_grad_inputs(inputs, dev):
    """Stand-in forward states and incoming gradients of the gated workload for
    the gradient pass (the pass is defined for any given states)."""
    cfg = inputs.GATED_LARGE
    B, T, N = cfg["B"], cfg["T"], cfg["N"]
    return {"s": inputs.random_normal((B, T, N), 2001).to(dev),
            "ds": inputs.random_normal((B, T, N), 2002).to(dev),
            "dsf": inputs.random_state((B, N), 2003).to(dev)}


def small_call_row(ctx, binding, dev, name, fn, fn_cabi, nbytes, units, unit, key):
    """A launch-bound call: host time per call through the binding and through
    the C ABI directly (enqueue only), GPU time per call from events over
    back-to-back calls and from a HIP graph of 100 calls, wall time per call,
    and the rocprofv3 kernel-only duration (current source only)."""
    import torch

    ms_call, ms_events = time_steps(fn, 200, 10)
    torch.cuda.synchronize()
    def host_us(f):
        f()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(100):
            f()
        dt = time.perf_counter() - t0
        torch.cuda.synchronize()
        return dt / 100 * 1e6
    us_host = host_us(fn)
    us_cabi = host_us(fn_cabi)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(100):
                fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us_graph = e0.elapsed_time(e1) * 1e3 / 500
    del g
    return {"row": name, "us_per_call": round(ms_call * 1e3, 3), "us_gpu_events": round(ms_events * 1e3, 3),
            "us_gpu_in_graph": round(us_graph, 3),
            "us_kernel_rocprof": measured_kernel_us(key, "scan_elem.hip"),
            "us_host_binding": round(us_host, 3), "us_host_cabi": round(us_cabi, 3),
            "host_share": round(us_host / (ms_call * 1e3), 3),
            f"{unit}_per_s": round(units / (ms_events * 1e-3), 1),
            "GB/s": round(nbytes / (ms_events * 1e-3) / 1e9, 2),
            "note": f"{nbytes / 1e6:.2f} MB per call: launch-latency bound; no roofline claim"}


def row_elem_small(kind, ctx, binding, inputs, dev, flush, copy):
    import ctypes

    import numpy as np
    import torch

    import oracle

    d = inputs.elementwise_small(**inputs.ELEM_SMALL)
    a = d["a"].to(dev)
    x = (d["b"] if kind == "fma" else d["u"]).to(dev)
    s = torch.empty_like(a)
    fin = torch.empty((a.shape[0], a.shape[2]), device=dev)
    f = binding.lrs_scan_fma if kind == "fma" else binding.lrs_scan_gated
    fn = lambda: f(ctx, a, x, None, s, fin)  # noqa: E731
    L = binding.lib()
    cf = L.lrs_scan_fma if kind == "fma" else L.lrs_scan_gated
    args = (ctx.handle, a.data_ptr(), x.data_ptr(), None, s.data_ptr(), fin.data_ptr(), 2, 128, 128,
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    fn_cabi = lambda: cf(*args)  # noqa: E731
    row = small_call_row(ctx, binding, dev, f"scan_{kind} B=2 T=128 N=128 fp32", fn, fn_cabi,
                         elem_bytes(2, 128, 128, with_s0=False), 2 * 128 * 128, "elements",
                         f"scan_elem_{kind}_B2_T128_N128")
    fn()
    torch.cuda.synchronize()
    ref = (oracle.scan_fma if kind == "fma" else oracle.scan_gated)(d["a"], d["b"] if kind == "fma" else d["u"])
    row["parity_max_rel_err"] = max(float(np.max(np.abs(s.cpu().numpy() - ref[0])) / np.max(np.abs(ref[0]))),
                                    float(np.max(np.abs(fin.cpu().numpy() - ref[1])) / np.max(np.abs(ref[1]))))
    row["inputs_sha256_16"] = digests(d, ("a", "b" if kind == "fma" else "u"))
    return row


def row_step_small(ctx, binding, inputs, dev, flush, copy):
    import ctypes

    import numpy as np
    import torch

    import oracle

    B, N = STEP_SMALL
    sd = inputs.elementwise_small(B, 1, N, seed=2010)
    sa, sx = sd["a"][:, 0].contiguous().to(dev), sd["u"][:, 0].contiguous().to(dev)
    st0 = inputs.random_state((B, N), 2011)
    st = st0.to(dev)
    binding.lrs_step_gated(ctx, sa, sx, st)
    torch.cuda.synchronize()
    ref = oracle.scan_gated(sd["a"], sd["u"], st0)[1]
    err = float(np.max(np.abs(st.cpu().numpy() - ref)) / np.max(np.abs(ref)))
    fn = lambda: binding.lrs_step_gated(ctx, sa, sx, st)  # noqa: E731
    L = binding.lib()
    args = (ctx.handle, sa.data_ptr(), sx.data_ptr(), st.data_ptr(), B, N,
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    fn_cabi = lambda: L.lrs_step_gated(*args)  # noqa: E731
    row = small_call_row(ctx, binding, dev, f"step_gated B={B} N={N} fp32 (one in-place decode step)", fn, fn_cabi,
                         16 * B * N, B * N, "channels", "step_elem_gated_B16_N2048")
    row["parity_max_rel_err"] = err
    row["inputs_sha256_16"] = {"a": inputs.digest(sd["a"]), "u": inputs.digest(sd["u"]), "s": inputs.digest(st0)}
    return row


def row_step_large(ctx, binding, inputs, dev, flush, copy):
    import torch

    sa = torch.full(STEP_LARGE, 0.75, device=dev)
    sx = torch.ones(STEP_LARGE, device=dev)
    st = torch.zeros(STEP_LARGE, device=dev)
    n = STEP_LARGE[0] * STEP_LARGE[1]
    fn = lambda: binding.lrs_step_gated(ctx, sa, sx, st)  # noqa: E731
    med, mn = time_launches(fn, 10, 2, flush)
    torch.cuda.synchronize()
    # twelve steps s <- 0.75 s + 0.25 from s = 0 leave s = 1 - 0.75^12 everywhere
    err = float((st - (1.0 - 0.75 ** 12)).abs().max().item())
    r = roofline(16 * n, med, copy)
    r["traffic"] = measured_traffic("step_elem_gated_B16_N4194304", "scan_elem.hip")
    return {"row": f"step_gated B={STEP_LARGE[0]} N={STEP_LARGE[1]} fp32 (one in-place step, 1 GiB stream)",
            "us_median": round(med * 1e3, 2), "us_min": round(mn * 1e3, 2), "roofline": r,
            "inputs": "constants a = 0.75, u = 1, s = 0", "max_abs_err_vs_closed_form": err}


def row_elem_bwd(kind, ctx, binding, inputs, dev, flush, copy):
    import numpy as np
    import torch

    import oracle

    cfg = inputs.GATED_LARGE
    B, T, N = cfg["B"], cfg["T"], cfg["N"]
    d = inputs.gated_large(**cfg)
    a, u, s0 = d["a"].to(dev), d["u"].to(dev), d["s0"].to(dev)
    g = elem_grad_inputs(inputs, dev)
    da = torch.empty_like(a)
    dx = torch.empty_like(a)
    ds0 = torch.empty_like(s0)
    if kind == "gated":
        fn = lambda: binding.lrs_scan_gated_backward(ctx, a, u, s0, g["s"], g["ds"], g["dsf"],  # noqa: E731
                                                     da, dx, ds0)
        per_elem = 24
    else:
        fn = lambda: binding.lrs_scan_fma_backward(ctx, a, s0, g["s"], g["ds"], g["dsf"], da, dx, ds0)  # noqa: E731
        per_elem = 20
    med, mn = time_launches(fn, 10, 2, flush)
    torch.cuda.synchronize()
    assert binding.lrs_context_check(ctx) == binding.LRS_OK
    nbytes = per_elem * B * T * N + 3 * 4 * B * N
    r = roofline(nbytes, med, copy)
    r["traffic"] = measured_traffic(f"scan_elem_{kind}_bwd_B16_T8192_N2048", "scan_elem.hip")
    row = {"row": f"scan_{kind}_backward B=16 T=8192 N=2048 fp32 (gradient pass: reads a, ds, s"
                  f"{', u' if kind == 'gated' else ''}; writes da, d{'u' if kind == 'gated' else 'b'}, ds0)",
           "us_median": round(med * 1e3, 2), "us_min": round(mn * 1e3, 2),
           "elements_per_s": round(B * T * N / (med * 1e-3), 1), "roofline": r}
    host = {k: v.cpu().numpy() for k, v in (("a", a), ("u", u), ("s", g["s"]), ("ds", g["ds"]))}
    host0 = {k: v.cpu().numpy() for k, v in (("s0", s0), ("dsf", g["dsf"]))}
    if kind == "gated":
        run = lambda nth, bb=slice(None): oracle.scan_gated_backward(  # noqa: E731
            host["a"][bb], host["u"][bb], host["s"][bb], host["ds"][bb], host0["s0"][bb], host0["dsf"][bb],
            nthreads=nth)
    else:
        run = lambda nth, bb=slice(None): oracle.scan_fma_backward(  # noqa: E731
            host["a"][bb], host["s"][bb], host["ds"][bb], host0["s0"][bb], host0["dsf"][bb], nthreads=nth)
    one = slice(0, 1)
    res, cpu = oracle_cpu(lambda nth: run(nth), lambda nth: run(nth, one), nbytes / 1e9, "GB/s",
                          "the whole workload (B=16,T=8192,N=2048), sequential fp64 oracle incl. fp32->fp64 "
                          "upcast, OpenMP over (batch, channel-block)",
                          "batch row 0 of the workload (1/16 of it), one thread", nbytes / B / 1e9)
    gpu = (da.cpu().numpy(), dx.cpu().numpy(), ds0.cpu().numpy())
    row["parity_max_rel_err"] = max(float(np.max(np.abs(x - y)) / np.max(np.abs(y))) for x, y in zip(gpu, res))
    row["cpu_baseline"] = cpu
    row["inputs_sha256_16"] = {"a": inputs.digest(d["a"]), "u": inputs.digest(d["u"]),
                               "s0": inputs.digest(d["s0"])}
    return row


def diag_bytes(d):
    """Algorithmic HBM bytes of one scan_diag_outer call (inputs read once,
    outputs written once, no initial state)."""
    q, v, g, ks = d["q"], d["v"], d["g"], d["k_scale"]
    B, T, Hg, K = q.shape
    H, V = v.shape[2], v.shape[3]
    n = 2 * q.numel() * 2 + v.numel() * 2 + g.numel() * 4 + (ks.numel() * 4 if ks is not None else 0)
    if d.get("k_scale_key") is not None:
        n += d["k_scale_key"].numel() * 4
    return n + B * T * H * V * 4 + B * H * K * V * 4


def delta_bytes(d, out_bytes=4):
    q, v, beta = d["q"], d["v"], d["beta"]
    B, T, H, K = q.shape
    V = v.shape[3]
    g = d["g"].numel() * 4 if "g" in d else 0   # the decayed form's per-key log-decay
    return 2 * q.numel() * 2 + v.numel() * 2 + beta.numel() * 4 + g + B * T * H * V * out_bytes + B * H * K * V * 4


def with_epilogue(inputs, d, epi):
    """A diag-outer workload plus the inputs of one output epilogue."""
    B, T, H, V = d["v"].shape
    d = dict(d)
    if epi == 2:   # LRS_EPILOGUE_NORM_GATE
        d.update(inputs.norm_gate_epilogue(B, T, H, V))
    else:
        d.update(inputs.skip_epilogue(H))
    d["epilogue"] = epi
    return d


def epilogue_call(binding, ctx, d, dev):
    """A closure running the fused-epilogue scan with a bf16 output, and its
    output tensors."""
    import torch

    q, k, v, g = (d[n].to(dev) for n in ("q", "k", "v", "g"))
    B, T, Hg, K = q.shape
    H, V = v.shape[2], v.shape[3]
    ks = None if d["k_scale"] is None else d["k_scale"].to(dev)
    z = d["gate"].to(dev) if "gate" in d else None
    w = d["norm_weight"].to(dev) if "norm_weight" in d else None
    dsk = d["d_skip"].to(dev) if "d_skip" in d else None
    o = torch.empty((B, T, H, V), device=dev, dtype=torch.bfloat16)
    fin = torch.empty((B, H, K, V), device=dev)

    def fn():
        binding.lrs_scan_diag_outer_epilogue(ctx, q, k, v, g, d["decay_mode"], ks, d["scale"], None, d["epilogue"],
                                             dsk, z, w, d.get("eps", 0.0), binding.LRS_DTYPE_BF16, o, fin)
    return fn, (o, fin)


def epilogue_bytes(d):
    """Algorithmic bytes of a fused-epilogue call with a bf16 output: the scan's
    inputs, the epilogue's inputs, a bf16 o and the fp32 final state."""
    B, T, H, V = d["v"].shape
    n = diag_bytes(d) - B * T * H * V * 4 + B * T * H * V * 2
    if "gate" in d:
        n += d["gate"].numel() * 2 + d["norm_weight"].numel() * 4
    if "d_skip" in d:
        n += d["d_skip"].numel() * 4
    return n


MATRIX_ROWS = {
    # name: (label, kind, generator, traffic keys, out dtype)
    "mamba2": ("scan_diag_outer Mamba-2 B=8 T=4096 H=24 P=64 N=128 (scalar decay, 1 group)", "diag", "mamba2",
               ["diag_outer_agg_mamba2_B8_T4096_H24_P64_N128", "diag_prefix_mamba2_B8_T4096_H24_P64_N128",
                "diag_outer_out_mamba2_B8_T4096_H24_P64_N128"], "f32"),
    "gla": ("scan_diag_outer GLA B=4 T=4096 H=4 K=128 V=128 (per-key decay)", "diag", "gla",
            ["diag_outer_agg_gla_B4_T4096_H4_K128_V128", "diag_prefix_gla_B4_T4096_H4_K128_V128",
             "diag_outer_out_gla_B4_T4096_H4_K128_V128"], "f32"),
    "hgrn2": ("scan_diag_outer HGRN2 B=4 T=4096 H=16 K=128 V=128 (per-key decay, key = 1 - forget gate)", "diag",
              "hgrn2", ["diag_outer_agg_hgrn2_B4_T4096_H16_K128_V128", "diag_prefix_hgrn2_B4_T4096_H16_K128_V128",
                        "diag_outer_out_hgrn2_B4_T4096_H16_K128_V128"], "f32"),
    "assoc": ("scan_diag_outer_keyscale associative memory B=4 T=4096 H=8 K=64 V=64 (per-key decay and kappa)",
              "keyscale", "assoc", ["diag_outer_agg_assoc_B4_T4096_H8_K64_V64",
                                    "diag_prefix_assoc_B4_T4096_H8_K64_V64",
                                    "diag_outer_out_assoc_B4_T4096_H8_K64_V64"], "f32"),
    "deltanet_k128": ("scan_delta DeltaNet B=4 T=4096 H=8 K=128 V=128", "delta", "deltanet",
                      ["delta_prep_deltanet_B4_T4096_H8_K128", "delta_scan_deltanet_B4_T4096_H8_K128_V128"], "f32"),
    "deltanet_k128_bf16": ("scan_delta_out DeltaNet B=4 T=4096 H=8 K=128 V=128, bf16 out", "delta", "deltanet",
                           ["delta_prep_deltanet_B4_T4096_H8_K128", "delta_scan_deltanet_B4_T4096_H8_K128_V128_bf16"],
                           "bf16"),
    "deltanet_k64": ("scan_delta DeltaNet B=4 T=4096 H=8 K=64 V=128", "delta", "deltanet_k64",
                     ["delta_prep_deltanet_B4_T4096_H8_K64", "delta_scan_deltanet_B4_T4096_H8_K64_V128"], "f32"),
    "rwkv7": ("scan_delta_decay RWKV-7 B=4 T=4096 H=12 K=64 V=64 (per-key decay)", "decay", "rwkv7",
              ["delta_prep_rwkv7_B4_T4096_H12_K64", "delta_scan_rwkv7_B4_T4096_H12_K64_V64"], "f32"),
    "rwkv7_bf16": ("scan_delta_out RWKV-7 B=4 T=4096 H=12 K=64 V=64 (per-key decay), bf16 out", "decay", "rwkv7",
                   ["delta_prep_rwkv7_B4_T4096_H12_K64", "delta_scan_rwkv7_B4_T4096_H12_K64_V64_bf16"], "bf16"),
    "decay_k128": ("scan_delta_decay B=4 T=4096 H=8 K=128 V=128 (per-key decay, RWKV-7's decay law)", "decay",
                   "decay_k128", ["delta_prep_decay_B4_T4096_H8_K128", "delta_scan_decay_B4_T4096_H8_K128_V128"],
                   "f32"),
    "decay_k128_bf16": ("scan_delta_out B=4 T=4096 H=8 K=128 V=128 (per-key decay), bf16 out", "decay",
                        "decay_k128", ["delta_prep_decay_B4_T4096_H8_K128",
                                       "delta_scan_decay_B4_T4096_H8_K128_V128_bf16"], "bf16"),
    # one long sequence: the automatic plan runs it in time segments (segment
    # pass, prefix over segments, output pass)
    "deltanet_b1_long": ("scan_delta DeltaNet B=1 T=16384 H=8 K=128 V=128 (time segments)", "delta",
                         "deltanet_b1_long",
                         ["delta_prep_deltanet_B1_T16384_H8_K128", "delta_segscan_deltanet_B1_T16384_H8_K128_V128",
                          "delta_segprefix_deltanet_B1_T16384_H8_K128_V128",
                          "delta_scan_deltanet_B1_T16384_H8_K128_V128"], "f32"),
}


def gen_workload(inputs, which):
    if which == "mamba2":
        return inputs.mamba2(**{k: v for k, v in inputs.MAMBA2.items() if k != "Hg"})
    return {"gla": lambda: inputs.gla(**inputs.GLA), "hgrn2": lambda: inputs.hgrn2(**inputs.HGRN2),
            "assoc": lambda: inputs.assoc_memory(**inputs.ASSOC),
            "deltanet": lambda: inputs.deltanet(**inputs.DELTANET),
            "deltanet_k64": lambda: inputs.deltanet(**inputs.DELTANET_K64),
            "rwkv7": lambda: inputs.rwkv7(**inputs.RWKV7),
            "decay_k128": lambda: inputs.rwkv7(**inputs.DELTA_DECAY_K128),
            "deltanet_b1_long": lambda: inputs.deltanet(**inputs.DELTANET_B1_LONG)}[which]()


def oracle_matrix(kind, d, nthreads, heads=None):
    """The fp64 oracle over the whole workload, or over the given (b, h) slices."""
    import oracle

    if heads is not None:
        outs = []
        for (bb, hh) in heads:
            sub = dict(d)
            grp = 0 if d["q"].shape[2] == 1 else hh
            for n in ("q", "k"):
                sub[n] = d[n][bb:bb + 1, :, grp:grp + 1]
            for n in ("v", "g", "beta", "k_scale", "k_scale_key"):
                if d.get(n) is not None and d[n].dim() >= 3:
                    sub[n] = d[n][bb:bb + 1, :, hh:hh + 1]
            outs.append(oracle_matrix(kind, sub, nthreads))
        return outs
    if kind in ("diag", "keyscale"):
        return oracle.scan_diag_outer(d["q"], d["k"], d["v"], d["g"], d["decay_mode"] if kind == "diag" else 1,
                                      d["k_scale"] if kind == "diag" else None, d["scale"], nthreads=nthreads,
                                      k_scale_key=d.get("k_scale_key") if kind == "keyscale" else None)
    if kind == "decay":
        return oracle.scan_delta_decay(d["q"], d["k"], d["v"], d["g"], d["beta"], d["scale"], nthreads=nthreads)
    return oracle.scan_delta(d["q"], d["k"], d["v"], d["beta"], d["scale"], nthreads=nthreads)


def row_matrix(name, ctx, binding, inputs, dev, flush, copy):
    import numpy as np
    import torch

    label, kind, which, traffic_keys, odt = MATRIX_ROWS[name]
    d = gen_workload(inputs, which)
    q, k, v = (d[n].to(dev) for n in ("q", "k", "v"))
    B, T = q.shape[0], q.shape[1]
    H, V, K = v.shape[2], v.shape[3], q.shape[3]
    bf = odt == "bf16"
    o = torch.empty((B, T, H, V), device=dev, dtype=torch.bfloat16 if bf else torch.float32)
    fin = torch.empty((B, H, K, V), device=dev)
    if kind == "diag":
        g = d["g"].to(dev)
        ks = None if d["k_scale"] is None else d["k_scale"].to(dev)
        fn = lambda: binding.lrs_scan_diag_outer(ctx, q, k, v, g, d["decay_mode"], ks, d["scale"],  # noqa: E731
                                                 None, o, fin)
        nbytes, flops_per_unit, src = diag_bytes(d), 5 * K * V, "scan_diag_outer.hip"
    elif kind == "keyscale":
        g, kk = d["g"].to(dev), d["k_scale_key"].to(dev)
        fn = lambda: binding.lrs_scan_diag_outer_keyscale(ctx, q, k, v, g, kk, d["scale"], None, o, fin)  # noqa: E731
        nbytes, flops_per_unit, src = diag_bytes(d), 5 * K * V, "scan_diag_outer.hip"
    else:
        beta = d["beta"].to(dev)
        g = d["g"].to(dev) if kind == "decay" else None
        dt = binding.LRS_DTYPE_BF16 if bf else binding.LRS_DTYPE_F32
        fn = lambda: binding.lrs_scan_delta_out(ctx, q, k, v, g, beta, d["scale"], None, dt, o, fin)  # noqa: E731
        nbytes, flops_per_unit, src = delta_bytes(d, 2 if bf else 4), 6 * K * V, "scan_delta.hip"
    med, mn = time_launches(fn, 20, 3, flush)
    torch.cuda.synchronize()
    units = B * T * H
    r = roofline(nbytes, med, copy)
    tr = [measured_traffic(key, src) for key in traffic_keys]
    r["traffic"] = None if any(t is None for t in tr) else sum(tr)
    row = {"row": label, "us_median": round(med * 1e3, 2), "us_min": round(mn * 1e3, 2),
           "tokens_heads_per_s": round(units / (med * 1e-3), 1), "roofline": r,
           "algorithmic_TFLOP/s": round(units * flops_per_unit / (med * 1e-3) / 1e12, 3),
           "mfma_util": measured_mfma_util(traffic_keys, src)}
    # parity on every (b, h) slice and the oracle over the whole workload
    heads1 = [(0, 0)]
    res, cpu = oracle_cpu(lambda nth: oracle_matrix(kind, d, nth), lambda nth: oracle_matrix(kind, d, nth, heads1),
                          units, "tokens*heads/s",
                          f"the whole workload ({B * H} (batch, head) slices x T={T}), fp64 oracle, OpenMP over "
                          "(batch, head)", "one (batch, head) slice x full T, one thread", T * len(heads1))
    ro, rf = res
    go = o.float().cpu().double().numpy()
    gf = fin.cpu().double().numpy()
    worst = 0.0
    for bb in range(B):
        for hh in range(H):
            eo = float(np.max(np.abs(go[bb, :, hh] - ro[bb, :, hh])) / np.max(np.abs(ro[bb, :, hh])))
            ef = float(np.max(np.abs(gf[bb, hh] - rf[bb, hh])) / np.max(np.abs(rf[bb, hh])))
            worst = max(worst, eo, ef)
    row["parity_max_rel_err_all_heads"] = worst
    if bf:
        row["parity_note"] = "bf16 output: tolerance 2e-3 + 2^-8 (the output's own rounding)"
    row["cpu_baseline"] = cpu
    row["inputs_sha256_16"] = digests(d, ("q", "k", "v", "g", "beta", "k_scale", "k_scale_key"))
    return row


EPI_ROWS = {
    "epi_gla": ("scan_diag_outer_epilogue GLA B=4 T=4096 H=4 K=128 V=128 + RMSNorm(o)*silu(gate), bf16 out", "gla", 2,
                ["diag_outer_agg_gla_B4_T4096_H4_K128_V128", "diag_prefix_gla_B4_T4096_H4_K128_V128",
                 "diag_outer_out_epi_normgate_gla_B4_T4096_H4_K128_V128"]),
    "epi_mamba2": ("scan_diag_outer_epilogue Mamba-2 B=8 T=4096 H=24 P=64 N=128 + D x skip, bf16 out", "mamba2", 1,
                   ["diag_outer_agg_mamba2_B8_T4096_H24_P64_N128", "diag_prefix_mamba2_B8_T4096_H24_P64_N128",
                    "diag_outer_out_epi_skip_mamba2_B8_T4096_H24_P64_N128"]),
}


def row_epilogue(name, ctx, binding, inputs, dev, flush, copy):
    import numpy as np
    import torch

    import oracle

    label, which, epi, traffic_keys = EPI_ROWS[name]
    d = with_epilogue(inputs, gen_workload(inputs, which), epi)
    fn, (o, fin) = epilogue_call(binding, ctx, d, dev)
    B, T, H, V = d["v"].shape
    K = d["q"].shape[3]
    med, mn = time_launches(fn, 20, 3, flush)
    torch.cuda.synchronize()
    nbytes = epilogue_bytes(d)
    units = B * T * H
    r = roofline(nbytes, med, copy)
    tr = [measured_traffic(key, "scan_diag_outer.hip") for key in traffic_keys]
    r["traffic"] = None if any(t is None for t in tr) else sum(tr)
    row = {"row": label, "us_median": round(med * 1e3, 2), "us_min": round(mn * 1e3, 2),
           "tokens_heads_per_s": round(units / (med * 1e-3), 1), "roofline": r,
           "algorithmic_TFLOP/s": round(units * 5 * K * V / (med * 1e-3) / 1e12, 3),
           "mfma_util": measured_mfma_util(traffic_keys, "scan_diag_outer.hip")}

    def full(nth, heads=None):
        ro, rf = oracle_matrix("diag", d, nth) if heads is None else oracle_matrix("diag", d, nth, heads)[0]
        sl = (slice(None),) if heads is None else (slice(0, 1), slice(None), slice(0, 1))
        if epi == 2:
            ro = oracle.epilogue_norm_gate(ro, d["gate"][sl] if heads is not None else d["gate"], d["norm_weight"],
                                           d["eps"])
        else:
            ro = oracle.epilogue_skip(ro, d["d_skip"][:1] if heads is not None else d["d_skip"],
                                      d["v"][sl] if heads is not None else d["v"])
        return ro, rf

    res, cpu = oracle_cpu(lambda nth: full(nth), lambda nth: full(nth, [(0, 0)]), units, "tokens*heads/s",
                          f"the whole workload ({B * H} slices x T={T}), scan then epilogue, fp64 oracle",
                          "one (batch, head) slice x full T, scan then epilogue, one thread", T)
    ro, rf = res
    go = o.float().cpu().double().numpy()
    gf = fin.cpu().double().numpy()
    row["parity_max_rel_err_all_heads"] = max(
        max(float(np.max(np.abs(go[bb, :, hh] - ro[bb, :, hh])) / np.max(np.abs(ro[bb, :, hh]))),
            float(np.max(np.abs(gf[bb, hh] - rf[bb, hh])) / np.max(np.abs(rf[bb, hh]))))
        for bb in range(B) for hh in range(H))
    row["parity_note"] = "bf16 output: tolerance 2e-3 + 2^-8 (the output's own rounding)"
    row["cpu_baseline"] = cpu
    row["inputs_sha256_16"] = digests(d, ("q", "k", "v", "g", "k_scale", "gate"))
    return row


def row_noalloc(ctx, binding, inputs, dev, flush, copy):
    import torch

    cfg = inputs.GATED_LARGE
    B, T, N = cfg["B"], cfg["T"], cfg["N"]
    d = inputs.gated_large(**cfg)
    a, u, s0 = d["a"].to(dev), d["u"].to(dev), d["s0"].to(dev)
    s = torch.empty_like(a)
    fin = torch.empty_like(s0)
    fn = lambda: binding.lrs_scan_gated_noalloc(a, u, s0, s, fin)  # noqa: E731
    med, mn = time_launches(fn, 10, 2, flush)
    torch.cuda.synchronize()
    s2 = torch.empty_like(a)
    f2 = torch.empty_like(s0)
    binding.lrs_scan_gated(ctx, a, u, s0, s2, f2)
    torch.cuda.synchronize()
    err = float(((s - s2).abs().max() / s2.abs().max()).item())
    nbytes = elem_bytes(B, T, N)
    return {"row": "scan_gated_noalloc B=16 T=8192 N=2048 fp32 (allocation-free entry, static look-back scratch)",
            "us_median": round(med * 1e3, 2), "us_min": round(mn * 1e3, 2), "roofline": roofline(nbytes, med, copy),
            "max_rel_diff_vs_lrs_scan_gated": err}


ROWS = {
    "scan_fma_small": lambda *a: row_elem_small("fma", *a),
    "scan_gated_small": lambda *a: row_elem_small("gated", *a),
    "step_small": row_step_small,
    "scan_gated_bwd": lambda *a: row_elem_bwd("gated", *a),
    "scan_fma_bwd": lambda *a: row_elem_bwd("fma", *a),
    "step_large": row_step_large,
    "noalloc": row_noalloc,
    **{n: (lambda n_: (lambda *a: row_matrix(n_, *a)))(n) for n in MATRIX_ROWS},
    **{n: (lambda n_: (lambda *a: row_epilogue(n_, *a)))(n) for n in EPI_ROWS},
}


def run_one_row(name):
    """Runs one row in this process and prints it as one JSON line."""
    import torch

    from linear_recurrence_scan_fma_amd import binding, inputs

    dev = torch.device("cuda:0")
    with binding.Context(0) as ctx:
        flush = torch.ones(512 * 1024 * 1024 // 4, device=dev)
        row = ROWS[name](ctx, binding, inputs, dev, flush, None)
        del flush
    print(json.dumps(row), flush=True)


def run_rows_in_subprocesses():
    """Every row in a child process of its own (the measurement of one row
    never shares a process, allocator or cache state with another)."""
    rows = []
    for name in ROWS:
        log(f"[bench] row {name}")
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--row", name], capture_output=True,
                           text=True, timeout=600)
        if r.stderr:
            sys.stderr.write(r.stderr[-2000:])
        line = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
        if r.returncode != 0 or not line:
            rows.append({"row": name, "error": f"exit {r.returncode}"})
            continue
        rows.append(json.loads(line[-1]))
    return rows


def profile_run(ctx, binding, inputs, dev, steps, manifest_path=None):
    """Each kernel at its workload shape, `steps` launches, for rocprofv3
    (kernel trace or counters).  The copy of a 1 GiB tensor reads and writes
    exactly 2^30 bytes each way and calibrates FETCH_SIZE / WRITE_SIZE.

    With `manifest_path`, writes the launch order as JSON: a list of groups
    {"keys": [...], "calls": n, "alg_bytes": {...}, "title": ...}; each call
    of a group dispatches one kernel per key, in order (the library's
    look-back status fills aside), so a trace's dispatches can be labelled
    by position."""
    import torch

    manifest = []

    def group(keys, calls, title, alg=None):
        manifest.append({"keys": list(keys), "calls": calls, "title": title, "alg_bytes": alg or {}})

    src = torch.ones(1 << 28, device=dev)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    del src, dst
    d = inputs.gated_large(**inputs.GATED_LARGE)
    a, u, s0 = d["a"].to(dev), d["u"].to(dev), d["s0"].to(dev)
    s = torch.empty_like(a)
    fin = torch.empty_like(s0)
    cfg = inputs.GATED_LARGE
    eb = elem_bytes(cfg["B"], cfg["T"], cfg["N"])
    group(["scan_elem_gated_B16_T8192_N2048"], steps, "gated elementwise scan B=16 T=8192 N=2048 fp32",
          {"scan_elem_gated_B16_T8192_N2048": eb})
    for _ in range(steps):
        binding.lrs_scan_gated(ctx, a, u, s0, s, fin)
    torch.cuda.synchronize()
    # the gradient pass of the same workload (both forms)
    g = elem_grad_inputs(inputs, dev)
    da = torch.empty_like(a)
    dx = torch.empty_like(a)
    ds0 = torch.empty_like(s0)
    group(["scan_elem_gated_bwd_B16_T8192_N2048"], steps,
          "gradient pass of the gated elementwise scan B=16 T=8192 N=2048 fp32")
    for _ in range(steps):
        binding.lrs_scan_gated_backward(ctx, a, u, s0, g["s"], g["ds"], g["dsf"], da, dx, ds0)
    group(["scan_elem_fma_bwd_B16_T8192_N2048"], steps,
          "gradient pass of the FMA elementwise scan B=16 T=8192 N=2048 fp32")
    for _ in range(steps):
        binding.lrs_scan_fma_backward(ctx, a, s0, g["s"], g["ds"], g["dsf"], da, dx, ds0)
    torch.cuda.synchronize()
    del a, u, s, d, g, da, dx
    # one large single step (a pure 16 B per channel stream)
    sa = torch.full(STEP_LARGE, 0.5, device=dev)
    sx = torch.ones(STEP_LARGE, device=dev)
    st = torch.zeros(STEP_LARGE, device=dev)
    group(["step_elem_gated_B16_N4194304"], steps, "one gated step over B=16 x N=4194304 channels fp32")
    for _ in range(steps):
        binding.lrs_step_gated(ctx, sa, sx, st)
    torch.cuda.synchronize()
    del sa, sx, st
    # the launch-bound calls: the small workload's two scans and a decode step
    e = inputs.elementwise_small(**inputs.ELEM_SMALL)
    ea, eb, eu = e["a"].to(dev), e["b"].to(dev), e["u"].to(dev)
    es = torch.empty_like(ea)
    ef = torch.empty((2, 128), device=dev)
    ssa = torch.full(STEP_SMALL, 0.5, device=dev)
    ssx = torch.ones(STEP_SMALL, device=dev)
    sst = torch.zeros(STEP_SMALL, device=dev)
    group(["scan_elem_fma_B2_T128_N128", "scan_elem_gated_B2_T128_N128", "step_elem_gated_B16_N2048"], steps,
          "the launch-bound calls: FMA and gated scans B=2 T=128 N=128, one gated step B=16 N=2048")
    for _ in range(steps):
        binding.lrs_scan_fma(ctx, ea, eb, None, es, ef)
        binding.lrs_scan_gated(ctx, ea, eu, None, es, ef)
        binding.lrs_step_gated(ctx, ssa, ssx, sst)
    torch.cuda.synchronize()
    for name in MATRIX_ROWS:
        label, kind, which, keys, odt = MATRIX_ROWS[name]
        m = gen_workload(inputs, which)
        q, k, v = (m[n].to(dev) for n in ("q", "k", "v"))
        B, T, H, V = v.shape
        K = q.shape[3]
        o = torch.empty((B, T, H, V), device=dev, dtype=torch.bfloat16 if odt == "bf16" else torch.float32)
        fin = torch.empty((B, H, K, V), device=dev)
        call_bytes = (diag_bytes(m) if kind in ("diag", "keyscale") else delta_bytes(m, 2 if odt == "bf16" else 4))
        group(keys, steps, label, {"call": call_bytes})
        for _ in range(steps):
            if kind == "diag":
                binding.lrs_scan_diag_outer(ctx, q, k, v, m["g"].to(dev), m["decay_mode"],
                                            None if m["k_scale"] is None else m["k_scale"].to(dev), m["scale"],
                                            None, o, fin)
            elif kind == "keyscale":
                binding.lrs_scan_diag_outer_keyscale(ctx, q, k, v, m["g"].to(dev), m["k_scale_key"].to(dev),
                                                     m["scale"], None, o, fin)
            else:
                binding.lrs_scan_delta_out(ctx, q, k, v, m["g"].to(dev) if kind == "decay" else None,
                                           m["beta"].to(dev), m["scale"], None,
                                           binding.LRS_DTYPE_BF16 if odt == "bf16" else binding.LRS_DTYPE_F32,
                                           o, fin)
        torch.cuda.synchronize()
    for name in EPI_ROWS:
        label, which, epi, keys = EPI_ROWS[name]
        m = with_epilogue(inputs, gen_workload(inputs, which), epi)
        fn, _ = epilogue_call(binding, ctx, m, dev)
        group(keys, steps, label, {"call": epilogue_bytes(m)})
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
    assert binding.lrs_context_check(ctx) == binding.LRS_OK
    if manifest_path:
        with open(manifest_path, "w") as f:
            json.dump(manifest, f, indent=1)
    log("[bench] profile run done")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-rows", action="store_true", help="headline only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--row", help="run one row in this process and print it (used by the full run)")
    ap.add_argument("--manifest", help="with --profile: write the launch order (JSON) here")
    ap.add_argument("--profile", action="store_true",
                    help="for rocprofv3 runs: launch each kernel a few times, plus a plain 1 GiB "
                         "device copy that calibrates the HBM byte counters; prints no JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the scans run on a single MI355X; the library "
              "has no multi-GPU path (batch and head slices are independent, so each GPU would "
              "run its own share).", flush=True)
        sys.exit(2)
    if args.row:
        run_one_row(args.row)
        return

    import numpy as np
    import torch

    from linear_recurrence_scan_fma_amd import binding, inputs

    if args.profile:
        dev = torch.device("cuda:0")
        with binding.Context(0) as ctx:
            profile_run(ctx, binding, inputs, dev, args.steps, args.manifest)
        return

    # the rows first, each in a child process started before this process
    # touches the GPU
    rows = None
    if not args.no_rows:
        rows = run_rows_in_subprocesses()

    dev = torch.device("cuda:0")
    ctx = binding.Context(0)
    copy = copy_gbs(dev)
    log(f"[bench] 1 GiB device copy: {copy:.0f} GB/s")

    # ---- headline: gated elementwise scan, B=16 T=8192 N=2048 --------------------
    cfg = inputs.GATED_LARGE
    B, T, N = cfg["B"], cfg["T"], cfg["N"]
    log(f"[bench] generating gated workload {cfg}")
    d = inputs.gated_large(**cfg)
    a, u, s0 = d["a"].to(dev), d["u"].to(dev), d["s0"].to(dev)
    s = torch.empty_like(a)
    fin = torch.empty_like(s0)

    def step():
        binding.lrs_scan_gated(ctx, a, u, s0, s, fin)

    log("[bench] timing headline")
    ms_step, ms_kernel = time_steps(step, args.steps, args.warmup)
    torch.cuda.synchronize()
    assert binding.lrs_context_check(ctx) == binding.LRS_OK
    nbytes = elem_bytes(B, T, N)
    value = nbytes / (ms_step * 1e-3) / 1e9
    achieved = nbytes / (ms_kernel * 1e-3) / 1e9
    traffic = measured_traffic("scan_elem_gated_B16_T8192_N2048", "scan_elem.hip")
    line = {
        "metric": "scan throughput: GB/s & % HBM peak (elementwise); tokens/s·head & MFMA util",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded: a=sigmoid(N(2,1)), u~N(0,1), s0~N(0,1))",
        "config": {"workload": "gated elementwise scan B=16 T=8192 N=2048 fp32 (outputs all s_t and s_T)",
                   "elements": B * T * N, "bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "frac_of_copy": round(achieved / copy, 4),
                     "copy_GB/s": round(copy, 1)},
        "elements_per_s": round(B * T * N / (ms_kernel * 1e-3), 1),
        "inputs_sha256_16": {"a": inputs.digest(d["a"]), "u": inputs.digest(d["u"]), "s0": inputs.digest(d["s0"])},
    }

    # parity of the timed configuration against the oracle (full tensor), and
    # the oracle timed with every granted thread and on one thread
    if not args.no_cpu:
        ah, uh, s0h = d["a"].numpy(), d["u"].numpy(), d["s0"].numpy()
        import oracle

        res, cpu = oracle_cpu(lambda nth: oracle.scan_gated(ah, uh, s0h, nthreads=nth),
                              lambda nth: oracle.scan_gated(ah[:1], uh[:1], s0h[:1], nthreads=nth),
                              nbytes / 1e9, "GB/s",
                              "the full headline workload (B=16,T=8192,N=2048), sequential fp64 oracle "
                              "incl. fp32->fp64 upcast, OpenMP over (batch, channel-block)",
                              "batch row 0 of the headline workload (1/16 of it), one thread", nbytes / B / 1e9)
        rs, rf = res
        line["cpu_baseline"] = cpu
        gs = s.cpu().numpy()
        line["parity_max_rel_err"] = float(np.max(np.abs(gs - rs)) / np.max(np.abs(rs)))
        del rs, gs
    del a, u, s

    if rows is not None:
        for r in rows:
            rf_ = r.get("roofline")
            if rf_ and "achieved" in rf_:
                rf_["frac_of_copy"] = round(rf_["achieved"] / copy, 4)
        line["rows"] = rows

    ctx.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
