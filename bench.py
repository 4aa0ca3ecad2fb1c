"""Throughput of the scan library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-rows] [--no-cpu]

Headline (the JSON line's `value`): the gated elementwise scan
s_t = a_t s_{t-1} + (1 - a_t) u_t on B=16, T=8192, N=2048 fp32 with an fp32
initial state, inputs resident in HBM.  One step = one lrs_scan_gated call over
that batch.  `value` is algorithmic GB/s (inputs read once, outputs written
once) over the wall-clock of K steps; `roofline.achieved` uses the average
kernel duration from HIP events recorded on the launch stream.

`rows` reports the other scans at their workload shapes (each timed with
per-launch events; before each launch a 512 MB read evicts the call's inputs
from the 256 MB last-level cache), each with its own roofline figure.

`cpu_baseline` is the sequential CPU oracle (fp64) timed on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
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
    """The rocprofv3 counter record of a kernel in profiles/traffic.json, if it
    was taken on the current kernel source; else None."""
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


def elem_bytes(B, T, N, with_s0=True):
    return 12 * B * T * N + 4 * B * N + (4 * B * N if with_s0 else 0)


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-rows", action="store_true", help="headline only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--profile", action="store_true",
                    help="for rocprofv3 runs: launch each kernel a few times, plus a plain 1 GiB "
                         "device copy that calibrates the HBM byte counters; prints no JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the scans run on a single MI355X; the library "
              "has no multi-GPU path (batch and head slices are independent, so each GPU would "
              "run its own share).", flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from linear_recurrence_scan_fma_amd import binding, inputs

    dev = torch.device("cuda:0")
    ctx = binding.Context(0)
    if args.profile:
        profile_run(ctx, binding, inputs, dev, args.steps)
        ctx.close()
        return

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
                     "traffic": traffic},
        "elements_per_s": round(B * T * N / (ms_kernel * 1e-3), 1),
    }

    # parity of the timed configuration against the oracle (full tensor)
    if not args.no_cpu:
        import oracle

        ah, uh, s0h = d["a"].numpy(), d["u"].numpy(), d["s0"].numpy()
        nth = oracle.default_threads()
        log(f"[bench] timing CPU oracle on the full workload with {nth} threads")
        t0 = time.perf_counter()
        rs, rf = oracle.scan_gated(ah, uh, s0h, nthreads=nth)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": nth, "kind": "oracle",
            "sample": "the full headline workload (B=16,T=8192,N=2048), sequential fp64 oracle "
                      "incl. fp32->fp64 upcast, OpenMP over (batch, channel-block)",
            "seconds": round(dt, 3)}
        gs = s.cpu().numpy()
        err = float(np.max(np.abs(gs - rs)) / np.max(np.abs(rs)))
        line["parity_max_rel_err"] = err
        del rs, gs
    del a, u, s

    if not args.no_rows:
        line["rows"] = run_rows(ctx, args, binding, inputs, dev)

    ctx.close()
    print(json.dumps(line), flush=True)


def profile_run(ctx, binding, inputs, dev, steps):
    """Each kernel at its workload shape, `steps` launches, for rocprofv3
    (kernel trace or counters).  The copy of a 1 GiB tensor reads and writes
    exactly 2^30 bytes each way and calibrates FETCH_SIZE / WRITE_SIZE."""
    import torch

    src = torch.ones(1 << 28, device=dev)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    del src, dst
    d = inputs.gated_large(**inputs.GATED_LARGE)
    a, u, s0 = d["a"].to(dev), d["u"].to(dev), d["s0"].to(dev)
    s = torch.empty_like(a)
    fin = torch.empty_like(s0)
    for _ in range(steps):
        binding.lrs_scan_gated(ctx, a, u, s0, s, fin)
    torch.cuda.synchronize()
    # the gradient pass of the same workload (both forms)
    g = elem_grad_inputs(inputs, dev)
    da = torch.empty_like(a)
    dx = torch.empty_like(a)
    ds0 = torch.empty_like(s0)
    for _ in range(steps):
        binding.lrs_scan_gated_backward(ctx, a, u, s0, g["s"], g["ds"], g["dsf"], da, dx, ds0)
    for _ in range(steps):
        binding.lrs_scan_fma_backward(ctx, a, s0, g["s"], g["ds"], g["dsf"], da, dx, ds0)
    torch.cuda.synchronize()
    del a, u, s, d, g, da, dx
    # one large single step (a pure 16 B per channel stream)
    sa = torch.full(STEP_LARGE, 0.5, device=dev)
    sx = torch.ones(STEP_LARGE, device=dev)
    st = torch.zeros(STEP_LARGE, device=dev)
    for _ in range(steps):
        binding.lrs_step_gated(ctx, sa, sx, st)
    torch.cuda.synchronize()
    del sa, sx, st
    for gen, kind in ((lambda: inputs.mamba2(**{k: v for k, v in inputs.MAMBA2.items() if k != "Hg"}), "diag"),
                      (lambda: inputs.gla(**inputs.GLA), "diag"),
                      (lambda: inputs.hgrn2(**inputs.HGRN2), "diag"),
                      (lambda: inputs.assoc_memory(**inputs.ASSOC), "keyscale"),
                      (lambda: inputs.deltanet(**inputs.DELTANET), "delta"),
                      (lambda: inputs.deltanet(**inputs.DELTANET_K64), "delta"),
                      (lambda: inputs.rwkv7(**inputs.RWKV7), "decay")):
        m = gen()
        q, k, v = (m[n].to(dev) for n in ("q", "k", "v"))
        for _ in range(steps):
            if kind == "diag":
                binding.scan_diag_outer(ctx, q, k, v, m["g"].to(dev), m["decay_mode"],
                                        None if m["k_scale"] is None else m["k_scale"].to(dev), m["scale"])
            elif kind == "decay":
                binding.scan_delta_decay(ctx, q, k, v, m["g"].to(dev), m["beta"].to(dev), m["scale"])
            elif kind == "keyscale":
                binding.scan_diag_outer_keyscale(ctx, q, k, v, m["g"].to(dev), m["k_scale_key"].to(dev), m["scale"])
            else:
                binding.scan_delta(ctx, q, k, v, m["beta"].to(dev), m["scale"])
        torch.cuda.synchronize()
    for gen, epi in ((lambda: inputs.gla(**inputs.GLA), binding.LRS_EPILOGUE_NORM_GATE),
                     (lambda: inputs.mamba2(**{k: v for k, v in inputs.MAMBA2.items() if k != "Hg"}),
                      binding.LRS_EPILOGUE_SKIP)):
        m = with_epilogue(inputs, gen(), epi)
        fn, _ = epilogue_call(binding, ctx, m, dev)
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
    assert binding.lrs_context_check(ctx) == binding.LRS_OK
    log("[bench] profile run done")


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


def elem_rows(ctx, binding, inputs, dev, flush):
    """The gradient pass of the gated workload (both forms) and the single
    step, each with a roofline figure, parity on sampled batch rows and the
    CPU oracle timed on the same sample."""
    import numpy as np
    import torch

    import oracle

    rows = []
    cfg = inputs.GATED_LARGE
    B, T, N = cfg["B"], cfg["T"], cfg["N"]
    log("[bench] row: gradient pass of the gated workload")
    d = inputs.gated_large(**cfg)
    a, u, s0 = d["a"].to(dev), d["u"].to(dev), d["s0"].to(dev)
    g = elem_grad_inputs(inputs, dev)
    da = torch.empty_like(a)
    dx = torch.empty_like(a)
    ds0 = torch.empty_like(s0)
    nth = oracle.default_threads()
    # parity and the CPU oracle on the whole workload
    host = {k: v.cpu().numpy() for k, v in (("a", a), ("u", u), ("s", g["s"]), ("ds", g["ds"]))}
    host0 = {k: v.cpu().numpy() for k, v in (("s0", s0), ("dsf", g["dsf"]))}
    for kind in ("gated", "fma"):
        if kind == "gated":
            fn = lambda: binding.lrs_scan_gated_backward(ctx, a, u, s0, g["s"], g["ds"], g["dsf"],  # noqa: E731
                                                         da, dx, ds0)
            per_elem = 24
        else:
            fn = lambda: binding.lrs_scan_fma_backward(ctx, a, s0, g["s"], g["ds"], g["dsf"],  # noqa: E731
                                                       da, dx, ds0)
            per_elem = 20
        med, mn = time_launches(fn, 10, 2, flush)
        torch.cuda.synchronize()
        assert binding.lrs_context_check(ctx) == binding.LRS_OK
        nbytes = per_elem * B * T * N + 3 * 4 * B * N
        achieved = nbytes / (med * 1e-3) / 1e9
        key = f"scan_elem_{kind}_bwd_B16_T8192_N2048"
        row = {"row": f"scan_{kind}_backward B=16 T=8192 N=2048 fp32 (gradient pass: reads a, ds, s"
                      f"{', u' if kind == 'gated' else ''}; writes da, d{'u' if kind == 'gated' else 'b'}, ds0)",
               "us_median": round(med * 1e3, 2), "us_min": round(mn * 1e3, 2),
               "elements_per_s": round(B * T * N / (med * 1e-3), 1),
               "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                            "bytes_per_call": nbytes,
                            "traffic": measured_traffic(key, "scan_elem.hip")}}
        t0 = time.perf_counter()
        if kind == "gated":
            r = oracle.scan_gated_backward(host["a"], host["u"], host["s"], host["ds"], host0["s0"],
                                           host0["dsf"], nthreads=nth)
        else:
            r = oracle.scan_fma_backward(host["a"], host["s"], host["ds"], host0["s0"], host0["dsf"],
                                         nthreads=nth)
        dt = time.perf_counter() - t0
        gpu = (da.cpu().numpy(), dx.cpu().numpy(), ds0.cpu().numpy())
        row["parity_max_rel_err"] = max(float(np.max(np.abs(x - y)) / np.max(np.abs(y))) for x, y in zip(gpu, r))
        del gpu, r
        row["cpu_baseline"] = {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s",
                               "cores": nth, "kind": "oracle",
                               "sample": "the whole workload (B=16,T=8192,N=2048), sequential fp64 oracle "
                                         "incl. fp32->fp64 upcast, OpenMP over (batch, channel-block)",
                               "seconds": round(dt, 3)}
        rows.append(row)
    del a, u, s0, g, da, dx, ds0, d, host, host0

    log("[bench] row: single step")
    for shape in (STEP_SMALL, STEP_LARGE):
        n = shape[0] * shape[1]
        sd = inputs.elementwise_small(shape[0], 1, shape[1], seed=2010) if n <= 1 << 20 else None
        if sd is not None:
            sa, sx = sd["a"][:, 0].to(dev), sd["u"][:, 0].to(dev)
        else:
            sa = torch.full(shape, 0.75, device=dev)
            sx = torch.ones(shape, device=dev)
        st0 = inputs.random_state(shape, 2011) if n <= 1 << 20 else None
        st = st0.to(dev) if st0 is not None else torch.zeros(shape, device=dev)
        if st0 is not None:
            # parity: one step against the oracle's one-step scan
            binding.lrs_step_gated(ctx, sa, sx, st)
            ref = oracle.scan_gated(sd["a"], sd["u"], st0)[1]
            err = float(np.max(np.abs(st.cpu().numpy() - ref)) / np.max(np.abs(ref)))
        fn = lambda: binding.lrs_step_gated(ctx, sa, sx, st)  # noqa: E731
        if n <= 1 << 20:
            ms_call, ms_kernel = time_steps(fn, 200, 10)
            row = {"row": f"step_gated B={shape[0]} N={shape[1]} fp32 (one in-place decode step)",
                   "us_per_call": round(ms_call * 1e3, 3), "us_kernel_events": round(ms_kernel * 1e3, 3),
                   "channels_per_s": round(n / (ms_kernel * 1e-3), 1),
                   "parity_max_rel_err": err,
                   "note": f"{16 * n / 1e6:.2f} MB per step: launch-latency bound; no roofline claim"}
        else:
            med, mn = time_launches(fn, 10, 2, flush)
            achieved = 16 * n / (med * 1e-3) / 1e9
            row = {"row": f"step_gated B={shape[0]} N={shape[1]} fp32 (one in-place step, 1 GiB stream)",
                   "us_median": round(med * 1e3, 2), "us_min": round(mn * 1e3, 2),
                   "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                                "bytes_per_call": 16 * n,
                                "traffic": measured_traffic("step_elem_gated_B16_N4194304", "scan_elem.hip")}}
        rows.append(row)
        del sa, sx, st
    return rows


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


def delta_bytes(d):
    q, v, beta = d["q"], d["v"], d["beta"]
    B, T, H, K = q.shape
    V = v.shape[3]
    g = d["g"].numel() * 4 if "g" in d else 0   # the decayed form's per-key log-decay
    return 2 * q.numel() * 2 + v.numel() * 2 + beta.numel() * 4 + g + B * T * H * V * 4 + B * H * K * V * 4


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


def run_rows(ctx, args, binding, inputs, dev):
    """The other scans at their workload shapes, each with a roofline figure,
    parity on sampled heads, and the CPU oracle timed on a sample beside it."""
    import numpy as np
    import torch

    import oracle

    rows = []
    # small elementwise workload (launch-latency bound; no roofline claim)
    d = inputs.elementwise_small(**inputs.ELEM_SMALL)
    a, b, u = d["a"].to(dev), d["b"].to(dev), d["u"].to(dev)
    for kind, x in (("fma", b), ("gated", u)):
        s = torch.empty_like(a)
        fin = torch.empty((a.shape[0], a.shape[2]), device=dev)
        fn = binding.lrs_scan_fma if kind == "fma" else binding.lrs_scan_gated
        ms_step, ms_kernel = time_steps(lambda: fn(ctx, a, x, None, s, fin), 200, 10)
        nbytes = elem_bytes(2, 128, 128, with_s0=False)
        rows.append({"row": f"scan_{kind} B=2 T=128 N=128 fp32", "us_per_call": round(ms_kernel * 1e3, 3),
                     "elements_per_s": round(32768 / (ms_kernel * 1e-3), 1),
                     "GB/s": round(nbytes / (ms_kernel * 1e-3) / 1e9, 2),
                     "note": "launch-latency bound (394 KB per call); no roofline claim"})

    flush = torch.ones(512 * 1024 * 1024 // 4, device=dev)
    rows += elem_rows(ctx, binding, inputs, dev, flush)
    nth = oracle.default_threads()
    heads = [(0, 0), (1, 1)]
    specs = [
        ("scan_diag_outer Mamba-2 B=8 T=4096 H=24 P=64 N=128 (scalar decay, 1 group)", "diag",
         lambda: inputs.mamba2(**{k: v for k, v in inputs.MAMBA2.items() if k != "Hg"}),
         ["diag_outer_agg_mamba2_B8_T4096_H24_P64_N128", "diag_prefix_mamba2_B8_T4096_H24_P64_N128",
          "diag_outer_out_mamba2_B8_T4096_H24_P64_N128"]),
        ("scan_diag_outer GLA B=4 T=4096 H=4 K=128 V=128 (per-key decay)", "diag",
         lambda: inputs.gla(**inputs.GLA),
         ["diag_outer_agg_gla_B4_T4096_H4_K128_V128", "diag_prefix_gla_B4_T4096_H4_K128_V128",
          "diag_outer_out_gla_B4_T4096_H4_K128_V128"]),
        ("scan_diag_outer HGRN2 B=4 T=4096 H=16 K=128 V=128 (per-key decay, key = 1 - forget gate)", "diag",
         lambda: inputs.hgrn2(**inputs.HGRN2),
         ["diag_outer_agg_hgrn2_B4_T4096_H16_K128_V128", "diag_prefix_hgrn2_B4_T4096_H16_K128_V128",
          "diag_outer_out_hgrn2_B4_T4096_H16_K128_V128"]),
        ("scan_diag_outer_keyscale associative memory B=4 T=4096 H=8 K=64 V=64 (per-key decay and kappa)",
         "keyscale", lambda: inputs.assoc_memory(**inputs.ASSOC),
         ["diag_outer_agg_assoc_B4_T4096_H8_K64_V64", "diag_prefix_assoc_B4_T4096_H8_K64_V64",
          "diag_outer_out_assoc_B4_T4096_H8_K64_V64"]),
        ("scan_delta DeltaNet B=4 T=4096 H=8 K=128 V=128", "delta", lambda: inputs.deltanet(**inputs.DELTANET),
         ["delta_prep_deltanet_B4_T4096_H8_K128", "delta_scan_deltanet_B4_T4096_H8_K128_V128"]),
        ("scan_delta DeltaNet B=4 T=4096 H=8 K=64 V=128", "delta", lambda: inputs.deltanet(**inputs.DELTANET_K64),
         ["delta_prep_deltanet_B4_T4096_H8_K64", "delta_scan_deltanet_B4_T4096_H8_K64_V128"]),
        ("scan_delta_decay RWKV-7 B=4 T=4096 H=12 K=64 V=64 (per-key decay)", "decay",
         lambda: inputs.rwkv7(**inputs.RWKV7),
         ["delta_prep_rwkv7_B4_T4096_H12_K64", "delta_scan_rwkv7_B4_T4096_H12_K64_V64"]),
    ]
    for name, kind, gen, traffic_keys in specs:
        log(f"[bench] row {name}")
        d = gen()
        q, k, v = (d[n].to(dev) for n in ("q", "k", "v"))
        B, T = q.shape[0], q.shape[1]
        H, V, K = v.shape[2], v.shape[3], q.shape[3]
        o = torch.empty((B, T, H, V), device=dev)
        fin = torch.empty((B, H, K, V), device=dev)
        if kind == "diag":
            g = d["g"].to(dev)
            ks = None if d["k_scale"] is None else d["k_scale"].to(dev)
            fn = lambda: binding.lrs_scan_diag_outer(ctx, q, k, v, g, d["decay_mode"], ks, d["scale"],  # noqa: E731
                                                     None, o, fin)
            nbytes = diag_bytes(d)
            flops_per_unit = 5 * K * V
        elif kind == "keyscale":
            g, kk = d["g"].to(dev), d["k_scale_key"].to(dev)
            fn = lambda: binding.lrs_scan_diag_outer_keyscale(ctx, q, k, v, g, kk, d["scale"], None, o, fin)  # noqa: E731
            nbytes = diag_bytes(d)
            flops_per_unit = 5 * K * V
        elif kind == "decay":
            beta, g = d["beta"].to(dev), d["g"].to(dev)
            fn = lambda: binding.lrs_scan_delta_decay(ctx, q, k, v, g, beta, d["scale"], None, o, fin)  # noqa: E731
            nbytes = delta_bytes(d)
            flops_per_unit = 6 * K * V
        else:
            beta = d["beta"].to(dev)
            fn = lambda: binding.lrs_scan_delta(ctx, q, k, v, beta, d["scale"], None, o, fin)  # noqa: E731
            nbytes = delta_bytes(d)
            flops_per_unit = 6 * K * V
        med, mn = time_launches(fn, 20, 3, flush)
        units = B * T * H
        row = {"row": name, "us_median": round(med * 1e3, 2), "us_min": round(mn * 1e3, 2),
               "tokens_heads_per_s": round(units / (med * 1e-3), 1),
               "roofline": {"bound": "hbm", "achieved": round(nbytes / (med * 1e-3) / 1e9, 2),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "bytes_per_call": nbytes},
               "algorithmic_TFLOP/s": round(units * flops_per_unit / (med * 1e-3) / 1e12, 3)}
        src = "scan_diag_outer.hip" if kind in ("diag", "keyscale") else "scan_delta.hip"
        tr = [measured_traffic(key, src) for key in traffic_keys]
        row["roofline"]["traffic"] = None if any(t is None for t in tr) else sum(tr)
        row["mfma_util"] = measured_mfma_util(traffic_keys, src)
        # parity and the CPU oracle on sampled heads (full time axis)
        errs = []
        t_cpu = 0.0
        for (bb, hh) in heads:
            if kind == "diag":
                grp = 0 if d["q"].shape[2] == 1 else hh
                sub = (d["q"][bb:bb + 1, :, grp:grp + 1], d["k"][bb:bb + 1, :, grp:grp + 1],
                       d["v"][bb:bb + 1, :, hh:hh + 1], d["g"][bb:bb + 1, :, hh:hh + 1], d["decay_mode"],
                       None if d["k_scale"] is None else d["k_scale"][bb:bb + 1, :, hh:hh + 1], d["scale"])
                t0 = time.perf_counter()
                ro, rf = oracle.scan_diag_outer(*sub, nthreads=1)
            elif kind == "keyscale":
                sub = tuple(d[n][bb:bb + 1, :, hh:hh + 1] for n in ("q", "k", "v", "g"))
                t0 = time.perf_counter()
                ro, rf = oracle.scan_diag_outer(*sub, 1, None, d["scale"], nthreads=1,
                                                k_scale_key=d["k_scale_key"][bb:bb + 1, :, hh:hh + 1])
            elif kind == "decay":
                sub = tuple(d[n][bb:bb + 1, :, hh:hh + 1] for n in ("q", "k", "v", "g", "beta"))
                t0 = time.perf_counter()
                ro, rf = oracle.scan_delta_decay(*sub, d["scale"], nthreads=1)
            else:
                sub = tuple(d[n][bb:bb + 1, :, hh:hh + 1] for n in ("q", "k", "v", "beta"))
                t0 = time.perf_counter()
                ro, rf = oracle.scan_delta(*sub, d["scale"], nthreads=1)
            t_cpu += time.perf_counter() - t0
            go = o[bb:bb + 1, :, hh:hh + 1].cpu().double().numpy()
            gf = fin[bb:bb + 1, hh:hh + 1].cpu().double().numpy()
            errs.append(max(float(np.max(np.abs(go - ro)) / np.max(np.abs(ro))),
                            float(np.max(np.abs(gf - rf)) / np.max(np.abs(rf)))))
        row["parity_max_rel_err_sampled_heads"] = max(errs)
        # heads are independent: one oracle thread per head gives nth heads in parallel
        row["cpu_baseline"] = {"value": round(len(heads) * T / t_cpu * min(nth, B * H), 1),
                               "unit": "tokens*heads/s", "cores": min(nth, B * H), "kind": "oracle",
                               "sample": f"{len(heads)} heads x full T timed on one thread (fp64 oracle), "
                                         f"scaled by the {min(nth, B * H)} threads the oracle spreads heads over"}
        rows.append(row)
        del q, k, v, o, fin

    # fused output epilogues with a bf16 output
    epi_specs = [
        ("scan_diag_outer_epilogue GLA B=4 T=4096 H=4 K=128 V=128 + RMSNorm(o)*silu(gate), bf16 out",
         lambda: inputs.gla(**inputs.GLA), binding.LRS_EPILOGUE_NORM_GATE,
         ["diag_outer_agg_gla_B4_T4096_H4_K128_V128", "diag_prefix_gla_B4_T4096_H4_K128_V128",
          "diag_outer_out_epi_normgate_gla_B4_T4096_H4_K128_V128"]),
        ("scan_diag_outer_epilogue Mamba-2 B=8 T=4096 H=24 P=64 N=128 + D x skip, bf16 out",
         lambda: inputs.mamba2(**{k: v for k, v in inputs.MAMBA2.items() if k != "Hg"}), binding.LRS_EPILOGUE_SKIP,
         ["diag_outer_agg_mamba2_B8_T4096_H24_P64_N128", "diag_prefix_mamba2_B8_T4096_H24_P64_N128",
          "diag_outer_out_epi_skip_mamba2_B8_T4096_H24_P64_N128"]),
    ]
    for name, gen, epi, traffic_keys in epi_specs:
        log(f"[bench] row {name}")
        d = with_epilogue(inputs, gen(), epi)
        fn, (o, fin) = epilogue_call(binding, ctx, d, dev)
        B, T, H, V = d["v"].shape
        K = d["q"].shape[3]
        med, mn = time_launches(fn, 20, 3, flush)
        nbytes = epilogue_bytes(d)
        units = B * T * H
        row = {"row": name, "us_median": round(med * 1e3, 2), "us_min": round(mn * 1e3, 2),
               "tokens_heads_per_s": round(units / (med * 1e-3), 1),
               "roofline": {"bound": "hbm", "achieved": round(nbytes / (med * 1e-3) / 1e9, 2),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "bytes_per_call": nbytes},
               "algorithmic_TFLOP/s": round(units * 5 * K * V / (med * 1e-3) / 1e12, 3)}
        tr = [measured_traffic(key, "scan_diag_outer.hip") for key in traffic_keys]
        row["roofline"]["traffic"] = None if any(t is None for t in tr) else sum(tr)
        row["mfma_util"] = measured_mfma_util(traffic_keys, "scan_diag_outer.hip")
        errs, t_cpu = [], 0.0
        for (bb, hh) in heads:
            grp = 0 if d["q"].shape[2] == 1 else hh
            sl = lambda x, c: x[bb:bb + 1, :, c:c + 1]  # noqa: E731
            t0 = time.perf_counter()
            ro, rf = oracle.scan_diag_outer(sl(d["q"], grp), sl(d["k"], grp), sl(d["v"], hh), sl(d["g"], hh),
                                            d["decay_mode"], None if d["k_scale"] is None else sl(d["k_scale"], hh),
                                            d["scale"], nthreads=1)
            if epi == binding.LRS_EPILOGUE_NORM_GATE:
                ro = oracle.epilogue_norm_gate(ro, sl(d["gate"], hh), d["norm_weight"], d["eps"])
            else:
                ro = oracle.epilogue_skip(ro, d["d_skip"][hh:hh + 1], sl(d["v"], hh))
            t_cpu += time.perf_counter() - t0
            go = o[bb:bb + 1, :, hh:hh + 1].float().cpu().double().numpy()
            gf = fin[bb:bb + 1, hh:hh + 1].cpu().double().numpy()
            errs.append(max(float(np.max(np.abs(go - ro)) / np.max(np.abs(ro))),
                            float(np.max(np.abs(gf - rf)) / np.max(np.abs(rf)))))
        row["parity_max_rel_err_sampled_heads"] = max(errs)
        row["parity_note"] = "bf16 output: tolerance 2e-3 + 2^-8 (the output's own rounding)"
        row["cpu_baseline"] = {"value": round(len(heads) * T / t_cpu * min(nth, B * H), 1),
                               "unit": "tokens*heads/s", "cores": min(nth, B * H), "kind": "oracle",
                               "sample": f"{len(heads)} heads x full T, scan then epilogue, one thread each "
                                         f"(fp64 oracle), scaled by {min(nth, B * H)} threads"}
        rows.append(row)
        del o, fin, d
    return rows


if __name__ == "__main__":
    main()
