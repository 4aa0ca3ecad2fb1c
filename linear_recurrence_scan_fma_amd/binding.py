"""Thin ctypes binding of liblrs.so, with the C ABI's own names.

Argument marshalling only: every function checks that the torch tensors it is
given are device tensors of the expected dtype and shape, derives the int32
dimensions from the shapes, and passes raw device pointers and the current
HIP stream to the C entry point of the same name.  All computation happens in
the library's HIP kernels.  If the library is not built, the first call
raises; there is no fallback.

    ctx = lrs_context_create(0)
    lrs_scan_gated(ctx, a, u, s0, s, s_final)        # enqueued on the current stream
    lrs_context_destroy(ctx)
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblrs.so")

# Mirrors of include/lrs_abi.h
LRS_ABI_VERSION_MAJOR = 1
LRS_OK, LRS_E_INVAL, LRS_E_NOMEM, LRS_E_IO, LRS_E_FORMAT, LRS_E_UNSUPPORTED, LRS_E_DEVICE = (
    0, -1, -2, -3, -4, -5, -6)
LRS_CAP_SCAN_FMA, LRS_CAP_SCAN_GATED, LRS_CAP_SCAN_DIAG_OUTER, LRS_CAP_SCAN_DELTA = 1, 2, 4, 8
LRS_CAP_ELEM_BACKWARD, LRS_CAP_ELEM_STEP, LRS_CAP_SCAN_DELTA_DECAY = 16, 32, 64
LRS_CAP_SCAN_DIAG_KEYSCALE, LRS_CAP_SCAN_DIAG_EPILOGUE, LRS_CAP_SCAN_DELTA_OUT = 128, 256, 512
LRS_EPILOGUE_NONE, LRS_EPILOGUE_SKIP, LRS_EPILOGUE_NORM_GATE = 0, 1, 2
LRS_DTYPE_F32, LRS_DTYPE_BF16 = 0, 1
LRS_PARAM_ELEM_SCHEDULE = 1
LRS_PARAM_DIAG_SEGMENTS = 2
LRS_PARAM_LOOKBACK_DELAY_SEED = 3
LRS_PARAM_DELTA_SEGMENTS = 4
LRS_ELEM_SCHEDULE_AUTO, LRS_ELEM_SCHEDULE_STREAM, LRS_ELEM_SCHEDULE_LOOKBACK = 0, 1, 2

# Every symbol the header declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_F = ctypes.c_float
SIGNATURES = {
    "lrs_abi_version": (_U32, []),
    "lrs_abi_check": (_I32, [_I32]),
    "lrs_abi_caps": (_U32, []),
    "lrs_status_string": (ctypes.c_char_p, [_I32]),
    "lrs_context_create": (_I32, [_I32, ctypes.POINTER(_P)]),
    "lrs_context_destroy": (None, [_P]),
    "lrs_context_set_param": (_I32, [_P, _I32, _I32]),
    "lrs_context_check": (_I32, [_P]),
    "lrs_scan_fma": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P]),
    "lrs_scan_gated": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P]),
    "lrs_scan_fma_backward": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P]),
    "lrs_scan_gated_backward": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       _I32, _I32, _I32, _P]),
    "lrs_step_fma": (_I32, [_P, _P, _P, _P, _I32, _I32, _P]),
    "lrs_step_gated": (_I32, [_P, _P, _P, _P, _I32, _I32, _P]),
    "lrs_scan_diag_outer": (_I32, [_P, _P, _P, _P, _P, _I32, _P, _F, _P, _P, _P,
                                   _I32, _I32, _I32, _I32, _I32, _I32, _P]),
    "lrs_scan_diag_outer_keyscale": (_I32, [_P, _P, _P, _P, _P, _P, _F, _P, _P, _P,
                                            _I32, _I32, _I32, _I32, _I32, _I32, _P]),
    "lrs_scan_diag_outer_epilogue": (_I32, [_P, _P, _P, _P, _P, _I32, _P, _F, _P, _I32, _P, _P, _P, _F,
                                            _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P]),
    "lrs_scan_delta": (_I32, [_P, _P, _P, _P, _P, _F, _P, _P, _P,
                              _I32, _I32, _I32, _I32, _I32, _P]),
    "lrs_scan_delta_decay": (_I32, [_P, _P, _P, _P, _P, _P, _F, _P, _P, _P,
                                    _I32, _I32, _I32, _I32, _I32, _P]),
    "lrs_scan_delta_out": (_I32, [_P, _P, _P, _P, _P, _P, _F, _P, _I32, _P, _P,
                                  _I32, _I32, _I32, _I32, _I32, _P]),
    "lrs_scan_gated_noalloc": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _P]),
}

_lib = None


class LrsError(RuntimeError):
    def __init__(self, name, status):
        self.status = status
        super().__init__(f"{name} failed: status {status} ({lrs_status_string(status)})")


def lib():
    """The loaded liblrs.so (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m linear_recurrence_scan_fma_amd.build` "
                "(or __graft_entry__.build()) first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _lib = handle
    return _lib


def _check(name, status):
    if status != LRS_OK:
        raise LrsError(name, status)


# ---- version / caps ----------------------------------------------------------
def lrs_abi_version() -> int:
    return lib().lrs_abi_version()


def lrs_abi_check(caller_major: int = LRS_ABI_VERSION_MAJOR) -> int:
    return lib().lrs_abi_check(caller_major)


def lrs_abi_caps() -> int:
    return lib().lrs_abi_caps()


def lrs_status_string(status: int) -> str:
    return lib().lrs_status_string(status).decode()


# ---- context -----------------------------------------------------------------
class Context:
    """Owns an LrsContext*; usable as a context manager."""

    def __init__(self, device: int = 0):
        h = _P()
        _check("lrs_context_create", lib().lrs_context_create(device, ctypes.byref(h)))
        self.handle = h
        self.device = device

    def close(self):
        if self.handle is not None and self.handle.value:
            lib().lrs_context_destroy(self.handle)
        self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def lrs_context_create(device: int = 0) -> Context:
    return Context(device)


def lrs_context_destroy(ctx: Context) -> None:
    ctx.close()


def lrs_context_set_param(ctx: Context, param: int, value: int) -> None:
    _check("lrs_context_set_param", lib().lrs_context_set_param(ctx.handle, param, value))


def lrs_context_check(ctx: Context) -> int:
    """Returns the status (does not raise): LRS_OK or LRS_E_DEVICE."""
    return lib().lrs_context_check(ctx.handle)


# ---- marshalling helpers -----------------------------------------------------
_Tensor = None


def _ptr(t, dtype, shape, name, device):
    # The checks use the cheapest tensor attributes (get_device() rather than
    # t.device): this runs for every tensor of every call, and small calls
    # (a decode step) are bounded by host time.
    global _Tensor
    if t is None:
        return None
    if _Tensor is None:
        import torch

        _Tensor = torch.Tensor
    if not isinstance(t, _Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.get_device() != device:
        raise ValueError(f"{name} must live on cuda:{device}, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_raw_stream = None


def _stream(stream, device):
    global _raw_stream
    if stream is None:
        if _raw_stream is None:
            import torch

            # the current stream's raw handle without building a Stream object
            _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None) or (
                lambda dev: torch.cuda.current_stream(dev).cuda_stream)
        return _raw_stream(device)
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---- scans -------------------------------------------------------------------
def _elem(name, ctx, a, x, s0, s, s_final, stream):
    import torch

    B, T, N = a.shape
    d = ctx.device
    f32 = torch.float32
    args = (
        _ptr(a, f32, (B, T, N), "a", d), _ptr(x, f32, (B, T, N), "b/u", d),
        _ptr(s0, f32, (B, N), "s0", d), _ptr(s, f32, (B, T, N), "s", d),
        _ptr(s_final, f32, (B, N), "s_final", d),
    )
    st = getattr(lib(), name)(ctx.handle, *args, B, T, N, _stream(stream, d))
    _check(name, st)


def lrs_scan_fma(ctx, a, b, s0, s, s_final, stream=None) -> None:
    """s_t = a_t s_{t-1} + b_t; a, b, s [B,T,N] fp32; s0 (or None), s_final [B,N]."""
    _elem("lrs_scan_fma", ctx, a, b, s0, s, s_final, stream)


def lrs_scan_gated(ctx, a, u, s0, s, s_final, stream=None) -> None:
    """s_t = a_t s_{t-1} + (1 - a_t) u_t; shapes as lrs_scan_fma."""
    _elem("lrs_scan_gated", ctx, a, u, s0, s, s_final, stream)


def lrs_scan_gated_noalloc(a, u, s0, s, s_final, stream=None) -> None:
    """lrs_scan_gated without a context or any allocation, on the tensors'
    device (which must be the current device); shapes as lrs_scan_gated."""
    import torch

    B, T, N = a.shape
    d = a.device.index if a.device.type == "cuda" else -1
    if d != torch.cuda.current_device():
        raise ValueError("lrs_scan_gated_noalloc runs on the current device: the tensors must live there")
    f32 = torch.float32
    args = (
        _ptr(a, f32, (B, T, N), "a", d), _ptr(u, f32, (B, T, N), "u", d),
        _ptr(s0, f32, (B, N), "s0", d), _ptr(s, f32, (B, T, N), "s", d),
        _ptr(s_final, f32, (B, N), "s_final", d),
    )
    st = lib().lrs_scan_gated_noalloc(*args, B, T, N, _stream(stream, d))
    _check("lrs_scan_gated_noalloc", st)


def lrs_scan_fma_backward(ctx, a, s0, s, ds, ds_final, da, db, ds0, stream=None) -> None:
    """Gradient pass of lrs_scan_fma: a, s, ds, da, db [B,T,N] fp32; s0,
    ds_final (None = zeros) and ds0 (None = not computed) [B,N] fp32."""
    import torch

    B, T, N = a.shape
    d = ctx.device
    f32 = torch.float32
    args = (
        _ptr(a, f32, (B, T, N), "a", d), _ptr(s0, f32, (B, N), "s0", d),
        _ptr(s, f32, (B, T, N), "s", d), _ptr(ds, f32, (B, T, N), "ds", d),
        _ptr(ds_final, f32, (B, N), "ds_final", d), _ptr(da, f32, (B, T, N), "da", d),
        _ptr(db, f32, (B, T, N), "db", d), _ptr(ds0, f32, (B, N), "ds0", d),
    )
    st = lib().lrs_scan_fma_backward(ctx.handle, *args, B, T, N, _stream(stream, d))
    _check("lrs_scan_fma_backward", st)


def lrs_scan_gated_backward(ctx, a, u, s0, s, ds, ds_final, da, du, ds0, stream=None) -> None:
    """Gradient pass of lrs_scan_gated; u, du [B,T,N] fp32, the rest as
    lrs_scan_fma_backward."""
    import torch

    B, T, N = a.shape
    d = ctx.device
    f32 = torch.float32
    args = (
        _ptr(a, f32, (B, T, N), "a", d), _ptr(u, f32, (B, T, N), "u", d),
        _ptr(s0, f32, (B, N), "s0", d), _ptr(s, f32, (B, T, N), "s", d),
        _ptr(ds, f32, (B, T, N), "ds", d), _ptr(ds_final, f32, (B, N), "ds_final", d),
        _ptr(da, f32, (B, T, N), "da", d), _ptr(du, f32, (B, T, N), "du", d),
        _ptr(ds0, f32, (B, N), "ds0", d),
    )
    st = lib().lrs_scan_gated_backward(ctx.handle, *args, B, T, N, _stream(stream, d))
    _check("lrs_scan_gated_backward", st)


def _step(name, ctx, a, x, s, stream):
    import torch

    B, N = a.shape
    d = ctx.device
    f32 = torch.float32
    args = (_ptr(a, f32, (B, N), "a", d), _ptr(x, f32, (B, N), "b/u", d), _ptr(s, f32, (B, N), "s", d))
    st = getattr(lib(), name)(ctx.handle, *args, B, N, _stream(stream, d))
    _check(name, st)


def lrs_step_fma(ctx, a, b, s, stream=None) -> None:
    """One step in place, s = a s + b; a, b, s [B,N] fp32."""
    _step("lrs_step_fma", ctx, a, b, s, stream)


def lrs_step_gated(ctx, a, u, s, stream=None) -> None:
    """One step in place, s = a s + (1 - a) u; a, u, s [B,N] fp32."""
    _step("lrs_step_gated", ctx, a, u, s, stream)


def lrs_scan_diag_outer(ctx, q, k, v, g, decay_mode, k_scale, scale, s0, o, s_final,
                        stream=None) -> None:
    """S_t = diag(exp(g_t)) S_{t-1} + (kappa_t k_t) v_t^T, o_t = scale S_t^T q_t.

    q, k [B,T,Hg,K] bf16; v [B,T,H,V] bf16; g [B,T,H] (mode 0) or [B,T,H,K]
    (mode 1) fp32; k_scale [B,T,H] fp32 or None; s0 [B,H,K,V] fp32 or None;
    o [B,T,H,V] fp32; s_final [B,H,K,V] fp32.
    """
    import torch

    B, T, Hg, K = q.shape
    H, V = v.shape[2], v.shape[3]
    d = ctx.device
    bf, f32 = torch.bfloat16, torch.float32
    gshape = (B, T, H) if decay_mode == 0 else (B, T, H, K)
    args = (
        _ptr(q, bf, (B, T, Hg, K), "q", d), _ptr(k, bf, (B, T, Hg, K), "k", d),
        _ptr(v, bf, (B, T, H, V), "v", d), _ptr(g, f32, gshape, "g", d), int(decay_mode),
        _ptr(k_scale, f32, (B, T, H), "k_scale", d), float(scale),
        _ptr(s0, f32, (B, H, K, V), "s0", d), _ptr(o, f32, (B, T, H, V), "o", d),
        _ptr(s_final, f32, (B, H, K, V), "s_final", d),
    )
    st = lib().lrs_scan_diag_outer(ctx.handle, *args, B, T, H, Hg, K, V, _stream(stream, d))
    _check("lrs_scan_diag_outer", st)


def lrs_scan_diag_outer_epilogue(ctx, q, k, v, g, decay_mode, k_scale, scale, s0, epilogue, d_skip, gate,
                                 norm_weight, eps, out_dtype, o, s_final, stream=None) -> None:
    """lrs_scan_diag_outer with a fused output epilogue (LRS_EPILOGUE_*) and an
    fp32 or bf16 output (LRS_DTYPE_*): d_skip [H] fp32; gate [B,T,H,V] bf16;
    norm_weight [V] fp32 or None; o [B,T,H,V] of out_dtype."""
    import torch

    B, T, Hg, K = q.shape
    H, V = v.shape[2], v.shape[3]
    d = ctx.device
    bf, f32 = torch.bfloat16, torch.float32
    gshape = (B, T, H) if decay_mode == 0 else (B, T, H, K)
    odt = bf if out_dtype == LRS_DTYPE_BF16 else f32
    args = (
        _ptr(q, bf, (B, T, Hg, K), "q", d), _ptr(k, bf, (B, T, Hg, K), "k", d),
        _ptr(v, bf, (B, T, H, V), "v", d), _ptr(g, f32, gshape, "g", d), int(decay_mode),
        _ptr(k_scale, f32, (B, T, H), "k_scale", d), float(scale),
        _ptr(s0, f32, (B, H, K, V), "s0", d), int(epilogue), _ptr(d_skip, f32, (H,), "d_skip", d),
        _ptr(gate, bf, (B, T, H, V), "gate", d), _ptr(norm_weight, f32, (V,), "norm_weight", d),
        float(eps), int(out_dtype), _ptr(o, odt, (B, T, H, V), "o", d),
        _ptr(s_final, f32, (B, H, K, V), "s_final", d),
    )
    st = lib().lrs_scan_diag_outer_epilogue(ctx.handle, *args, B, T, H, Hg, K, V, _stream(stream, d))
    _check("lrs_scan_diag_outer_epilogue", st)


def lrs_scan_diag_outer_keyscale(ctx, q, k, v, g, k_scale, scale, s0, o, s_final, stream=None) -> None:
    """As lrs_scan_diag_outer with per-key decay g [B,T,H,K] and per-key kappa
    k_scale [B,T,H,K] fp32 (required)."""
    import torch

    B, T, Hg, K = q.shape
    H, V = v.shape[2], v.shape[3]
    d = ctx.device
    bf, f32 = torch.bfloat16, torch.float32
    args = (
        _ptr(q, bf, (B, T, Hg, K), "q", d), _ptr(k, bf, (B, T, Hg, K), "k", d),
        _ptr(v, bf, (B, T, H, V), "v", d), _ptr(g, f32, (B, T, H, K), "g", d),
        _ptr(k_scale, f32, (B, T, H, K), "k_scale", d), float(scale),
        _ptr(s0, f32, (B, H, K, V), "s0", d), _ptr(o, f32, (B, T, H, V), "o", d),
        _ptr(s_final, f32, (B, H, K, V), "s_final", d),
    )
    st = lib().lrs_scan_diag_outer_keyscale(ctx.handle, *args, B, T, H, Hg, K, V, _stream(stream, d))
    _check("lrs_scan_diag_outer_keyscale", st)


def lrs_scan_delta(ctx, q, k, v, beta, scale, s0, o, s_final, stream=None) -> None:
    """delta_t = beta_t (v_t - S^T k_t), S += k_t delta_t^T, o_t = scale S_t^T q_t.

    q, k [B,T,H,K] bf16; v [B,T,H,V] bf16; beta [B,T,H] fp32; s0 [B,H,K,V] fp32
    or None; o [B,T,H,V] fp32; s_final [B,H,K,V] fp32.
    """
    import torch

    B, T, H, K = q.shape
    V = v.shape[3]
    d = ctx.device
    bf, f32 = torch.bfloat16, torch.float32
    args = (
        _ptr(q, bf, (B, T, H, K), "q", d), _ptr(k, bf, (B, T, H, K), "k", d),
        _ptr(v, bf, (B, T, H, V), "v", d), _ptr(beta, f32, (B, T, H), "beta", d),
        float(scale), _ptr(s0, f32, (B, H, K, V), "s0", d), _ptr(o, f32, (B, T, H, V), "o", d),
        _ptr(s_final, f32, (B, H, K, V), "s_final", d),
    )
    st = lib().lrs_scan_delta(ctx.handle, *args, B, T, H, K, V, _stream(stream, d))
    _check("lrs_scan_delta", st)


def lrs_scan_delta_decay(ctx, q, k, v, g, beta, scale, s0, o, s_final, stream=None) -> None:
    """delta_t = beta_t (v_t - S^T k_t), S = diag(exp(g_t)) S + k_t delta_t^T,
    o_t = scale S_t^T q_t.  As lrs_scan_delta plus g [B,T,H,K] fp32."""
    import torch

    B, T, H, K = q.shape
    V = v.shape[3]
    d = ctx.device
    bf, f32 = torch.bfloat16, torch.float32
    args = (
        _ptr(q, bf, (B, T, H, K), "q", d), _ptr(k, bf, (B, T, H, K), "k", d),
        _ptr(v, bf, (B, T, H, V), "v", d), _ptr(g, f32, (B, T, H, K), "g", d),
        _ptr(beta, f32, (B, T, H), "beta", d), float(scale), _ptr(s0, f32, (B, H, K, V), "s0", d),
        _ptr(o, f32, (B, T, H, V), "o", d), _ptr(s_final, f32, (B, H, K, V), "s_final", d),
    )
    st = lib().lrs_scan_delta_decay(ctx.handle, *args, B, T, H, K, V, _stream(stream, d))
    _check("lrs_scan_delta_decay", st)


def lrs_scan_delta_out(ctx, q, k, v, g, beta, scale, s0, out_dtype, o, s_final, stream=None) -> None:
    """lrs_scan_delta (g None) or lrs_scan_delta_decay (g [B,T,H,K] fp32) with the
    output o [B,T,H,V] written as out_dtype (LRS_DTYPE_F32: fp32 tensor,
    LRS_DTYPE_BF16: bf16 tensor)."""
    import torch

    B, T, H, K = q.shape
    V = v.shape[3]
    d = ctx.device
    bf, f32 = torch.bfloat16, torch.float32
    odt = bf if out_dtype == LRS_DTYPE_BF16 else f32
    args = (
        _ptr(q, bf, (B, T, H, K), "q", d), _ptr(k, bf, (B, T, H, K), "k", d),
        _ptr(v, bf, (B, T, H, V), "v", d), _ptr(g, f32, (B, T, H, K), "g", d),
        _ptr(beta, f32, (B, T, H), "beta", d), float(scale), _ptr(s0, f32, (B, H, K, V), "s0", d),
        int(out_dtype), _ptr(o, odt, (B, T, H, V), "o", d), _ptr(s_final, f32, (B, H, K, V), "s_final", d),
    )
    st = lib().lrs_scan_delta_out(ctx.handle, *args, B, T, H, K, V, _stream(stream, d))
    _check("lrs_scan_delta_out", st)


# ---- allocating conveniences (still marshalling only) -------------------------
def scan_elementwise(ctx, kind, a, x, s0=None, stream=None):
    """Allocates s and s_final and runs lrs_scan_fma (kind 'fma') or lrs_scan_gated."""
    import torch

    s = torch.empty_like(a)
    s_final = torch.empty((a.shape[0], a.shape[2]), dtype=a.dtype, device=a.device)
    fn = lrs_scan_fma if kind == "fma" else lrs_scan_gated
    fn(ctx, a, x, s0, s, s_final, stream)
    return s, s_final


def scan_elementwise_backward(ctx, kind, a, x, s, ds, s0=None, ds_final=None, stream=None):
    """Allocates da, dx, ds0 and runs the gradient pass of scan_elementwise
    (x = b for kind 'fma', unused there; x = u for 'gated').  Returns (da, dx, ds0)."""
    import torch

    da = torch.empty_like(a)
    dx = torch.empty_like(a)
    ds0 = torch.empty((a.shape[0], a.shape[2]), dtype=a.dtype, device=a.device)
    if kind == "fma":
        lrs_scan_fma_backward(ctx, a, s0, s, ds, ds_final, da, dx, ds0, stream)
    else:
        lrs_scan_gated_backward(ctx, a, x, s0, s, ds, ds_final, da, dx, ds0, stream)
    return da, dx, ds0


def scan_diag_outer(ctx, q, k, v, g, decay_mode, k_scale=None, scale=1.0, s0=None, stream=None):
    import torch

    B, T, Hg, K = q.shape
    H, V = v.shape[2], v.shape[3]
    o = torch.empty((B, T, H, V), dtype=torch.float32, device=q.device)
    fin = torch.empty((B, H, K, V), dtype=torch.float32, device=q.device)
    lrs_scan_diag_outer(ctx, q, k, v, g, decay_mode, k_scale, scale, s0, o, fin, stream)
    return o, fin


def scan_delta(ctx, q, k, v, beta, scale=1.0, s0=None, stream=None):
    import torch

    B, T, H, K = q.shape
    V = v.shape[3]
    o = torch.empty((B, T, H, V), dtype=torch.float32, device=q.device)
    fin = torch.empty((B, H, K, V), dtype=torch.float32, device=q.device)
    lrs_scan_delta(ctx, q, k, v, beta, scale, s0, o, fin, stream)
    return o, fin


def scan_delta_decay(ctx, q, k, v, g, beta, scale=1.0, s0=None, stream=None):
    import torch

    B, T, H, K = q.shape
    V = v.shape[3]
    o = torch.empty((B, T, H, V), dtype=torch.float32, device=q.device)
    fin = torch.empty((B, H, K, V), dtype=torch.float32, device=q.device)
    lrs_scan_delta_decay(ctx, q, k, v, g, beta, scale, s0, o, fin, stream)
    return o, fin


def scan_diag_outer_keyscale(ctx, q, k, v, g, k_scale, scale=1.0, s0=None, stream=None):
    import torch

    B, T, Hg, K = q.shape
    H, V = v.shape[2], v.shape[3]
    o = torch.empty((B, T, H, V), dtype=torch.float32, device=q.device)
    fin = torch.empty((B, H, K, V), dtype=torch.float32, device=q.device)
    lrs_scan_diag_outer_keyscale(ctx, q, k, v, g, k_scale, scale, s0, o, fin, stream)
    return o, fin


def scan_diag_outer_epilogue(ctx, q, k, v, g, decay_mode, k_scale=None, scale=1.0, s0=None,
                             epilogue=0, d_skip=None, gate=None, norm_weight=None, eps=1e-6,
                             out_dtype=0, stream=None):
    import torch

    B, T, Hg, K = q.shape
    H, V = v.shape[2], v.shape[3]
    odt = torch.bfloat16 if out_dtype == LRS_DTYPE_BF16 else torch.float32
    o = torch.empty((B, T, H, V), dtype=odt, device=q.device)
    fin = torch.empty((B, H, K, V), dtype=torch.float32, device=q.device)
    lrs_scan_diag_outer_epilogue(ctx, q, k, v, g, decay_mode, k_scale, scale, s0, epilogue, d_skip, gate,
                                 norm_weight, eps, out_dtype, o, fin, stream)
    return o, fin


def scan_delta_out(ctx, q, k, v, beta, g=None, scale=1.0, s0=None, out_dtype=LRS_DTYPE_BF16, stream=None):
    import torch

    B, T, H, K = q.shape
    V = v.shape[3]
    odt = torch.bfloat16 if out_dtype == LRS_DTYPE_BF16 else torch.float32
    o = torch.empty((B, T, H, V), dtype=odt, device=q.device)
    fin = torch.empty((B, H, K, V), dtype=torch.float32, device=q.device)
    lrs_scan_delta_out(ctx, q, k, v, g, beta, scale, s0, out_dtype, o, fin, stream)
    return o, fin
