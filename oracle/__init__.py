"""Sequential CPU reference for the linear-recurrence scans.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import this package.  It shares no code
with the GPU library and never calls it; the GPU library never calls this.

The arithmetic lives in ``lrs_oracle.c`` (plain C, no fast-math, no FMA
contraction).  This module only compiles it, loads it with ctypes and
marshals numpy arrays.  Every function returns new arrays in the requested
precision (``np.float64`` by default; ``np.float32`` runs the same loops in
single precision).

Sources, cited by short name:
  [SunnyNet log]  "SunnyNet 工程化实录：一个 O(N) 架构如何长出自己的 C 推理运行时",
                  developer.aliyun.com/article/1773847
  [vs llama.cpp]  "我拿同一份权重和 llama.cpp 正面比了一场：我手写的 C 内核，慢了 1.1–1.7 倍",
                  developer.aliyun.com/article/1775078
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lrs_oracle.c")
_SO = os.path.join(_HERE, "liblrs_oracle.so")
_lib = None


def build() -> str:
    """Compile the C oracle in place and return the path of the shared library."""
    cmd = [
        "gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
        "-shared", "-fPIC", "-std=c11", "-Wall", "-Wextra",
        _SRC, "-o", _SO + ".tmp", "-lm",
    ]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def default_threads() -> int:
    """Host threads the oracle may use: the threads this process is granted.
    That is OMP_NUM_THREADS when the environment sets it (a host's share of
    its cores for one job, which can be far below what the machine shows),
    else the whole affinity set; never more than the affinity set."""
    aff = max(1, len(os.sched_getaffinity(0)))
    env = os.environ.get("OMP_NUM_THREADS", "").strip()
    if env.isdigit() and int(env) > 0:
        return min(aff, int(env))
    return aff


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    for sfx in ("_f64", "_f32"):
        R = ctypes.c_double if sfx == "_f64" else ctypes.c_float
        for name in ("orc_scan_fma", "orc_scan_gated"):
            f = getattr(lib, name + sfx)
            f.argtypes = [P, P, P, P, P, I64, I64, I64, I]
            f.restype = None
        f = getattr(lib, "orc_scan_fma_bwd" + sfx)
        f.argtypes = [P, P, P, P, P, P, P, P, I64, I64, I64, I]
        f.restype = None
        f = getattr(lib, "orc_scan_gated_bwd" + sfx)
        f.argtypes = [P, P, P, P, P, P, P, P, P, I64, I64, I64, I]
        f.restype = None
        f = getattr(lib, "orc_scan_diag_outer" + sfx)
        f.argtypes = [P, P, P, P, I, P, P, R, P, P, P, I64, I64, I64, I64, I64, I64, I]
        f.restype = None
        for name in ("orc_scan_delta", "orc_scan_delta_explicit"):
            f = getattr(lib, name + sfx)
            f.argtypes = [P, P, P, P, R, P, P, P, I64, I64, I64, I64, I64, I]
            f.restype = None
        for name in ("orc_scan_delta_decay", "orc_scan_delta_decay_explicit"):
            f = getattr(lib, name + sfx)
            f.argtypes = [P, P, P, P, P, R, P, P, P, I64, I64, I64, I64, I64, I]
            f.restype = None
    lib.orc_version.restype = ctypes.c_int
    _lib = lib
    return lib


def version() -> int:
    return _load().orc_version()


def _sfx(dtype) -> str:
    dtype = np.dtype(dtype)
    if dtype == np.float64:
        return "_f64"
    if dtype == np.float32:
        return "_f32"
    raise ValueError(f"oracle precision must be float64 or float32, got {dtype}")


def _arr(x, dtype):
    """C-contiguous copy/view of ``x`` in ``dtype`` (exact for fp32/bf16 -> fp64)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: upcast on the host, exactly
        import torch

        x = x.detach().to("cpu", torch.float64 if np.dtype(dtype) == np.float64 else torch.float32).numpy()
    return np.ascontiguousarray(np.asarray(x), dtype=dtype)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _check_shape(name, x, shape):
    if x is not None and tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(x.shape)}")


def _elementwise(kind, a, x, s0, dtype, nthreads):
    a = _arr(a, dtype)
    x = _arr(x, dtype)
    if a.ndim != 3:
        raise ValueError("a must be [B,T,N]")
    B, T, N = a.shape
    _check_shape("b/u", x, (B, T, N))
    s0 = _arr(s0, dtype)
    _check_shape("s0", s0, (B, N))
    s = np.empty((B, T, N), dtype=dtype)
    fin = np.empty((B, N), dtype=dtype)
    fn = getattr(_load(), kind + _sfx(dtype))
    fn(_ptr(a), _ptr(x), _ptr(s0), _ptr(s), _ptr(fin), B, T, N, nthreads or default_threads())
    return s, fin


def scan_fma(a, b, s0=None, dtype=np.float64, nthreads=None):
    """s_t = a_t s_{t-1} + b_t over [B,T,N] inputs [SunnyNet log §2.1].

    Returns ``(s, s_final)`` with ``s[:, t-1] = s_t`` and ``s_final = s_T``.
    """
    return _elementwise("orc_scan_fma", a, b, s0, dtype, nthreads)


def scan_gated(a, u, s0=None, dtype=np.float64, nthreads=None):
    """s_t = a_t s_{t-1} + (1 - a_t) u_t over [B,T,N] inputs [SunnyNet log §2.1]."""
    return _elementwise("orc_scan_gated", a, u, s0, dtype, nthreads)


def _elementwise_bwd(gated, a, u, s0, s, ds, ds_final, dtype, nthreads):
    a = _arr(a, dtype)
    if a.ndim != 3:
        raise ValueError("a must be [B,T,N]")
    B, T, N = a.shape
    s = _arr(s, dtype)
    ds = _arr(ds, dtype)
    _check_shape("s", s, (B, T, N))
    _check_shape("ds", ds, (B, T, N))
    s0 = _arr(s0, dtype)
    _check_shape("s0", s0, (B, N))
    ds_final = _arr(ds_final, dtype)
    _check_shape("ds_final", ds_final, (B, N))
    da = np.empty((B, T, N), dtype=dtype)
    dx = np.empty((B, T, N), dtype=dtype)
    ds0 = np.empty((B, N), dtype=dtype)
    nth = nthreads or default_threads()
    if gated:
        u = _arr(u, dtype)
        _check_shape("u", u, (B, T, N))
        fn = getattr(_load(), "orc_scan_gated_bwd" + _sfx(dtype))
        fn(_ptr(a), _ptr(u), _ptr(s0), _ptr(s), _ptr(ds), _ptr(ds_final), _ptr(da), _ptr(dx),
           _ptr(ds0), B, T, N, nth)
    else:
        fn = getattr(_load(), "orc_scan_fma_bwd" + _sfx(dtype))
        fn(_ptr(a), _ptr(s0), _ptr(s), _ptr(ds), _ptr(ds_final), _ptr(da), _ptr(dx), _ptr(ds0),
           B, T, N, nth)
    return da, dx, ds0


def scan_fma_backward(a, s, ds, s0=None, ds_final=None, dtype=np.float64, nthreads=None):
    """Reverse (gradient) pass of ``scan_fma`` [SunnyNet log §8, reverse-scan entry].

    ``s`` are the forward states, ``ds`` the loss gradient with respect to each
    of them and ``ds_final`` with respect to the returned final state.
    gs_t = ds_t + a_{t+1} gs_{t+1} (gs_T = ds_T + ds_final); returns
    ``(da, db, ds0)`` with da_t = gs_t s_{t-1}, db_t = gs_t, ds0 = a_1 gs_1.
    """
    return _elementwise_bwd(False, a, None, s0, s, ds, ds_final, dtype, nthreads)


def scan_gated_backward(a, u, s, ds, s0=None, ds_final=None, dtype=np.float64, nthreads=None):
    """Reverse (gradient) pass of ``scan_gated``: as ``scan_fma_backward`` but
    da_t = gs_t (s_{t-1} - u_t) and du_t = gs_t (1 - a_t); returns ``(da, du, ds0)``."""
    return _elementwise_bwd(True, a, u, s0, s, ds, ds_final, dtype, nthreads)


def scan_diag_outer(q, k, v, g, decay_mode, k_scale=None, scale=1.0, s0=None,
                    dtype=np.float64, nthreads=None, k_scale_key=None):
    """Decay-separable outer-product state scan with readout.

    S_t = diag(exp(g_t)) S_{t-1} + (kappa_t k_t) v_t^T,  o_t = scale S_t^T q_t
    [SunnyNet log §4.1 (Mamba-2), §4.3 (GLA)].  Shapes: q, k [B,T,Hg,K];
    v [B,T,H,V]; g [B,T,H] (mode 0) or [B,T,H,K] (mode 1); k_scale [B,T,H];
    s0 [B,H,K,V].  ``k_scale_key`` [B,T,H,K] (instead of k_scale) scales each
    key: the matrix associative memory [vs llama.cpp §8] with g = log p and
    kappa = 1 - p.  Returns ``(o [B,T,H,V], s_final [B,H,K,V])``.
    """
    q, k, v, g = (_arr(x, dtype) for x in (q, k, v, g))
    B, T, Hg, K = q.shape
    H, V = v.shape[2], v.shape[3]
    _check_shape("k", k, (B, T, Hg, K))
    _check_shape("v", v, (B, T, H, V))
    if H % Hg:
        raise ValueError("H must be a multiple of Hg")
    if decay_mode not in (0, 1):
        raise ValueError("decay_mode must be 0 or 1")
    _check_shape("g", g, (B, T, H) if decay_mode == 0 else (B, T, H, K))
    k_scale = _arr(k_scale, dtype)
    _check_shape("k_scale", k_scale, (B, T, H))
    k_scale_key = _arr(k_scale_key, dtype)
    _check_shape("k_scale_key", k_scale_key, (B, T, H, K))
    if k_scale is not None and k_scale_key is not None:
        raise ValueError("give k_scale or k_scale_key, not both")
    s0 = _arr(s0, dtype)
    _check_shape("s0", s0, (B, H, K, V))
    o = np.empty((B, T, H, V), dtype=dtype)
    fin = np.empty((B, H, K, V), dtype=dtype)
    fn = getattr(_load(), "orc_scan_diag_outer" + _sfx(dtype))
    fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), int(decay_mode), _ptr(k_scale), _ptr(k_scale_key),
       float(scale), _ptr(s0), _ptr(o), _ptr(fin), B, T, H, Hg, K, V, nthreads or default_threads())
    return o, fin


def _delta(name, q, k, v, beta, scale, s0, dtype, nthreads):
    q, k, v, beta = (_arr(x, dtype) for x in (q, k, v, beta))
    B, T, H, K = q.shape
    V = v.shape[3]
    _check_shape("k", k, (B, T, H, K))
    _check_shape("v", v, (B, T, H, V))
    _check_shape("beta", beta, (B, T, H))
    s0 = _arr(s0, dtype)
    _check_shape("s0", s0, (B, H, K, V))
    o = np.empty((B, T, H, V), dtype=dtype)
    fin = np.empty((B, H, K, V), dtype=dtype)
    fn = getattr(_load(), name + _sfx(dtype))
    fn(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), float(scale), _ptr(s0), _ptr(o), _ptr(fin),
       B, T, H, K, V, nthreads or default_threads())
    return o, fin


def scan_delta(q, k, v, beta, scale=1.0, s0=None, dtype=np.float64, nthreads=None):
    """Delta rule, rank-1 form [SunnyNet log §4.2]:
    delta_t = beta_t (v_t - S_{t-1}^T k_t), S_t = S_{t-1} + k_t delta_t^T,
    o_t = scale S_t^T q_t.  Shapes: q, k [B,T,H,K]; v [B,T,H,V]; beta [B,T,H].
    """
    return _delta("orc_scan_delta", q, k, v, beta, scale, s0, dtype, nthreads)


def scan_delta_explicit(q, k, v, beta, scale=1.0, s0=None, dtype=np.float64, nthreads=None):
    """Delta rule, explicit form S_t = (I - beta k k^T) S_{t-1} + beta k v^T
    [SunnyNet log §4.2], implemented separately from the rank-1 form."""
    return _delta("orc_scan_delta_explicit", q, k, v, beta, scale, s0, dtype, nthreads)


def _delta_decay(name, q, k, v, g, beta, scale, s0, dtype, nthreads):
    q, k, v, g, beta = (_arr(x, dtype) for x in (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[3]
    _check_shape("k", k, (B, T, H, K))
    _check_shape("g", g, (B, T, H, K))
    _check_shape("v", v, (B, T, H, V))
    _check_shape("beta", beta, (B, T, H))
    s0 = _arr(s0, dtype)
    _check_shape("s0", s0, (B, H, K, V))
    o = np.empty((B, T, H, V), dtype=dtype)
    fin = np.empty((B, H, K, V), dtype=dtype)
    fn = getattr(_load(), name + _sfx(dtype))
    fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(s0), _ptr(o), _ptr(fin),
       B, T, H, K, V, nthreads or default_threads())
    return o, fin


def scan_delta_decay(q, k, v, g, beta, scale=1.0, s0=None, dtype=np.float64, nthreads=None):
    """Delta rule with a per-key decay, rank-1 form [SunnyNet log §5.1, RWKV-7]:
    delta_t = beta_t (v_t - S_{t-1}^T k_t), S_t = diag(exp(g_t)) S_{t-1} + k_t delta_t^T,
    o_t = scale S_t^T q_t.  Shapes: q, k, g [B,T,H,K]; v [B,T,H,V]; beta [B,T,H].
    """
    return _delta_decay("orc_scan_delta_decay", q, k, v, g, beta, scale, s0, dtype, nthreads)


def scan_delta_decay_explicit(q, k, v, g, beta, scale=1.0, s0=None, dtype=np.float64, nthreads=None):
    """The same update as a dense transition S_t = (diag(exp(g_t)) - beta k k^T) S_{t-1}
    + beta k v^T [SunnyNet log §5.1], implemented separately from the rank-1 form."""
    return _delta_decay("orc_scan_delta_decay_explicit", q, k, v, g, beta, scale, s0, dtype, nthreads)


# ---- output epilogues (plain numpy definitions, float64) -----------------------
def epilogue_norm_gate(o, z, weight=None, eps=1e-6):
    """GLA's output epilogue [SunnyNet log §4.3]: normalise first, then gate.

    out[b,t,h,:] = o / sqrt(mean_j o[b,t,h,j]^2 + eps) * weight * silu(z[b,t,h,:]),
    silu(x) = x / (1 + exp(-x)); RMSNorm over the value axis of each head;
    ``weight`` [V] (None: ones).  o, z [B,T,H,V].
    """
    o = np.asarray(o, dtype=np.float64)
    z = _arr(z, np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    w = np.ones(o.shape[-1]) if weight is None else _arr(weight, np.float64)
    return o / np.sqrt(ms + eps) * w * (z / (1.0 + np.exp(-z)))


def epilogue_skip(o, d_skip, x):
    """Mamba-2's skip connection: out[b,t,h,:] = o[b,t,h,:] + D[h] x[b,t,h,:],
    with x the scan's value input.  o, x [B,T,H,V]; D [H]."""
    o = np.asarray(o, dtype=np.float64)
    return o + _arr(d_skip, np.float64)[None, None, :, None] * _arr(x, np.float64)
