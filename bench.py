"""Throughput of the scan library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-rows] [--no-cpu]

Headline (the JSON line's `value`): the gated elementwise scan
s_t = a_t s_{t-1} + (1 - a_t) u_t on B=16, T=8192, N=2048 fp32 with an fp32
initial state, inputs resident in HBM.  One step = one lrs_scan_gated call over
that batch.  `value` is algorithmic GB/s (inputs read once, outputs written
once) over the wall-clock of K steps; `roofline.achieved` uses the average
kernel duration from HIP events recorded on the launch stream.

`rows` reports the other scans at their workload shapes (each timed with
per-launch events; the 256 MB last-level cache is flushed between launches of
the matrix scans), each with its own roofline figure.

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


def measured_traffic(kernel_key, source_file):
    """HBM bytes per launch measured by rocprofv3 counters, if the record in
    profiles/traffic.json was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec or rec.get("source_sha") != source_sha(source_file):
        return None
    return rec.get("bytes_per_launch")


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
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the scans run on a single MI355X and this "
              "build has no multi-GPU path (see DESIGN.md for how it would shard).", flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from linear_recurrence_scan_fma_amd import binding, inputs

    dev = torch.device("cuda:0")
    ctx = binding.Context(0)

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
    traffic = measured_traffic("scan_elem_gated_stream_16x8192x2048", "scan_elem.hip")
    line = {
        "metric": "gated elementwise scan throughput (algorithmic HBM GB/s)",
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


def run_rows(ctx, args, binding, inputs, dev):
    """The other scans at their workload shapes."""
    import torch

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
        rows.append({"row": f"scan_{kind} B=2 T=128 N=128", "us_per_call": round(ms_kernel * 1e3, 3),
                     "GB/s": round(nbytes / (ms_kernel * 1e-3) / 1e9, 2),
                     "note": "launch-latency bound (394 KB per call)"})
    return rows


if __name__ == "__main__":
    main()
