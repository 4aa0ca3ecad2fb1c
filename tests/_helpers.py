"""Shared helpers for the GPU parity tests (no method arithmetic here)."""
import sys

import numpy as np
import torch


def rel(x, y):
    """Normwise relative error max|x - y| / max|y| (max|x - y| when y == 0)."""
    x = x.detach().cpu().double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, np.float64)
    y = y.detach().cpu().double().numpy() if isinstance(y, torch.Tensor) else np.asarray(y, np.float64)
    if x.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    d = float(np.max(np.abs(x - y)))
    m = float(np.max(np.abs(y)))
    return d / m if m > 0 else d


def rel_heads(x, y, layout):
    """Max over (b, h) slices of the normwise relative error, so one bad head
    cannot hide behind the others.  layout: "bthv" ([B,T,H,V] outputs) or
    "bhkv" ([B,H,K,V] states).  A slice with fewer than 16 elements (a K = V = 1
    state is a single number, possibly ~0) is not a matrix and has no useful
    normwise error of its own; such tensors are compared normwise as a whole."""
    x = x.detach().cpu().double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, np.float64)
    y = y.detach().cpu().double().numpy() if isinstance(y, torch.Tensor) else np.asarray(y, np.float64)
    per_slice = x[0, :, 0].size if layout == "bthv" else x[0, 0].size
    if per_slice < 16:
        return rel(x, y)
    B = x.shape[0]
    H = x.shape[2] if layout == "bthv" else x.shape[1]
    worst = 0.0
    for b in range(B):
        for h in range(H):
            xs = x[b, :, h] if layout == "bthv" else x[b, h]
            ys = y[b, :, h] if layout == "bthv" else y[b, h]
            worst = max(worst, rel(xs, ys))
    return worst


def say(msg):
    """Progress line, flushed, so a GPU log names the case that ran last."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev(t):
    return None if t is None else t.to("cuda:0", non_blocking=False).contiguous()
