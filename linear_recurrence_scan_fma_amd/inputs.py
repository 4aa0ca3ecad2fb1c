"""Seeded synthetic inputs for the scan workloads.

This module holds no recurrence arithmetic.  It draws the inputs that both the
GPU library and the CPU reference consume, so the two sides always see exactly
the same values.  Every generator returns host (CPU) torch tensors, except the
``*_device`` ones at the end: for tensors of several GiB (the cases past
32-bit offsets) host draws would take minutes, so those follow the same
recipes with torch's seeded device generator, in float32, and return device
tensors (their values depend on the seed and on torch's generator).

Recipe (all draws from ``numpy.random.default_rng(seed)``; transcendentals in
float64; rounding to float32 by round-to-nearest-even; bfloat16 values are
float64 -> float32 -> bfloat16, each step round-to-nearest-even):

* elementwise, small:  a ~ U(0.5, 1), b ~ N(0, 1), u ~ N(0, 1), s0 = none, [B,T,N]
* elementwise, gated:  a = sigmoid(z), z ~ N(2, 1); u ~ N(0, 1); s0 ~ N(0, 1)
* gradient pass:       incoming gradients ds, ds_final ~ N(0, 1); at the full
                       size the forward states it reads are stand-in N(0, 1)
                       draws (the pass is defined for any given states)
* Mamba-2 shaped:      dt = softplus(N(0,1)) [B,T,H]; A_h = -exp(U(0,2)) [H];
                       g = dt * A_h (one log-decay per head and step);
                       B, C ~ N(0,1) bf16 [B,T,1,K]; x ~ N(0,1) bf16 [B,T,H,V]
* GLA shaped:          q, k, v ~ N(0,1) bf16 [B,T,H,D]; gk = logsigmoid(N(0,1))/16
                       fp32 [B,T,H,K]; readout scale K**-0.5
* DeltaNet shaped:     q, k = row-L2-normalised N(0,1), bf16 [B,T,H,K];
                       v ~ N(0,1) bf16 [B,T,H,V]; beta = sigmoid(N(0,1)) fp32 [B,T,H]
* associative memory:  q, k, v ~ N(0,1) bf16 [B,T,H,D]; p = sigmoid(N(2,1)) per
                       key fp32 [B,T,H,K]; g = log p, kappa = 1 - p (each from p
                       in float64); readout scale 1
* HGRN2 shaped:        f = sigmoid(N(2,1)) per key; g = log f fp32; k = 1 - f
                       bf16 (the key is tied to the forget gate); q, v ~ N(0,1)
                       bf16; readout scale 1
* output epilogues:    GLA norm-gate: gate z ~ N(0,1) bf16 [B,T,H,V], norm weight
                       ~ U(0.5,1.5) fp32 [V], eps 1e-6; Mamba-2 skip: D ~ U(0.5,1.5) [H]
* RWKV-7 shaped:       as DeltaNet, plus a per-key log-decay
                       g = -exp(-softplus(-z) - 0.5), z ~ N(0,1), fp32 [B,T,H,K]
                       (each step keeps a fraction in (0.545, 1) of every key row)

Model shapes follow the models named on the pages: Mamba-2 130m (24 heads x 64,
state 128) [SunnyNet log §4.1]; GLA 340M (4 heads x 128) [SunnyNet log §4.3];
DeltaNet 340M (8 heads x 128) [SunnyNet log §4.2]; RWKV-7 191M (64 x 64 state per
head, 12 heads) [SunnyNet log §5.1]; HGRN2 1.3B (dim 2048, 16 heads) ["我拿同一份权重和
llama.cpp 正面比了一场" §4].  The associative memory's shape is not given on the pages.  SunnyNet log =
"SunnyNet 工程化实录：一个 O(N) 架构如何长出自己的 C 推理运行时" (developer.aliyun.com/article/1773847).
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch

SEED_BASE = 1000  # config i uses SEED_BASE + i

# Full workload sizes (one GPU).
ELEM_SMALL = dict(B=2, T=128, N=128)
GATED_LARGE = dict(B=16, T=8192, N=2048)
MAMBA2 = dict(B=8, T=4096, H=24, Hg=1, K=128, V=64)
GLA = dict(B=4, T=4096, H=4, K=128, V=128)
DELTANET = dict(B=4, T=4096, H=8, K=128, V=128)
DELTANET_K64 = dict(B=4, T=4096, H=8, K=64, V=128)
RWKV7 = dict(B=4, T=4096, H=12, K=64, V=64)
DELTA_DECAY_K128 = dict(B=4, T=4096, H=8, K=128, V=128)   # RWKV-7's decay law at DeltaNet's head shape
HGRN2 = dict(B=4, T=4096, H=16, K=128, V=128)
ASSOC = dict(B=4, T=4096, H=8, K=64, V=64)
# one long DeltaNet sequence: too few (head, V-tile) workgroups to fill the
# chip, so the call splits the time axis into segments
DELTANET_B1_LONG = dict(B=1, T=16384, H=8, K=128, V=128)


def _f32(x64: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))


def _bf16(x64: np.ndarray) -> torch.Tensor:
    return _f32(x64).to(torch.bfloat16)


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _softplus(z):
    return np.logaddexp(0.0, z)


def _logsigmoid(z):
    return -np.logaddexp(0.0, -z)


def digest(t: torch.Tensor) -> str:
    """sha256 (first 16 hex digits) of a tensor's bytes, for logging inputs."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return hashlib.sha256(t.numpy().tobytes()).hexdigest()[:16]


def elementwise_small(B=2, T=128, N=128, seed=SEED_BASE + 1):
    """a ~ U(0.5,1), b ~ N(0,1), u ~ N(0,1), fp32 [B,T,N]; no initial state."""
    rng = np.random.default_rng(seed)
    a = rng.uniform(0.5, 1.0, size=(B, T, N))
    b = rng.standard_normal((B, T, N))
    u = rng.standard_normal((B, T, N))
    return dict(a=_f32(a), b=_f32(b), u=_f32(u), s0=None)


def gated_large(B=16, T=8192, N=2048, seed=SEED_BASE + 2, with_s0=True):
    """a = sigmoid(z), z ~ N(2,1); u ~ N(0,1); s0 ~ N(0,1); fp32 [B,T,N].

    Drawn one batch row at a time so the float64 temporaries stay small.
    """
    rng = np.random.default_rng(seed)
    a = torch.empty((B, T, N), dtype=torch.float32)
    u = torch.empty((B, T, N), dtype=torch.float32)
    for b in range(B):
        z = rng.standard_normal((T, N)) + 2.0
        a[b] = _f32(_sigmoid(z))
        del z
        u[b] = _f32(rng.standard_normal((T, N)))
    s0 = _f32(rng.standard_normal((B, N))) if with_s0 else None
    return dict(a=a, u=u, s0=s0)


def mamba2(B=8, T=4096, H=24, K=128, V=64, seed=SEED_BASE + 3):
    """Mamba-2 shaped decay-separable scan, one B/C group (Hg = 1).

    Mapping onto the scan: q = C, k = B, v = x, g = dt*A (one value per head and
    step, decay mode 0), k_scale = dt, readout scale 1.
    """
    rng = np.random.default_rng(seed)
    dt = _softplus(rng.standard_normal((B, T, H)))
    A = -np.exp(rng.uniform(0.0, 2.0, size=(H,)))
    dt32 = np.asarray(dt, dtype=np.float32)
    A32 = np.asarray(A, dtype=np.float32)
    g = dt32.astype(np.float64) * A32.astype(np.float64)[None, None, :]
    Bm = rng.standard_normal((B, T, 1, K))
    Cm = rng.standard_normal((B, T, 1, K))
    x = rng.standard_normal((B, T, H, V))
    return dict(q=_bf16(Cm), k=_bf16(Bm), v=_bf16(x), g=_f32(g), decay_mode=0,
                k_scale=_f32(dt32), scale=1.0, s0=None, A=_f32(A32))


def gla(B=4, T=4096, H=4, K=128, V=128, seed=SEED_BASE + 4):
    """GLA shaped scan: per-key decay gk = logsigmoid(N(0,1))/16 (decay mode 1)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    gk = _logsigmoid(rng.standard_normal((B, T, H, K))) / 16.0
    return dict(q=_bf16(q), k=_bf16(k), v=_bf16(v), g=_f32(gk), decay_mode=1,
                k_scale=None, scale=float(K) ** -0.5, s0=None)


def deltanet(B=4, T=4096, H=8, K=128, V=128, seed=SEED_BASE + 5):
    """DeltaNet shaped delta-rule scan: L2-normalised q, k; beta = sigmoid(N(0,1))."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V))
    beta = _sigmoid(rng.standard_normal((B, T, H)))
    return dict(q=_bf16(q), k=_bf16(k), v=_bf16(v), beta=_f32(beta), scale=1.0, s0=None)


def rwkv7(B=4, T=4096, H=12, K=64, V=64, seed=SEED_BASE + 6):
    """RWKV-7 shaped decayed delta rule: DeltaNet's q, k, v, beta plus a
    per-key log-decay bounded in (-exp(-0.5), 0)."""
    d = deltanet(B=B, T=T, H=H, K=K, V=V, seed=seed)
    rng = np.random.default_rng(seed + 1000)
    z = rng.standard_normal((B, T, H, K))
    d["g"] = _f32(-np.exp(-_softplus(-z) - 0.5))
    return d


def assoc_memory(B=4, T=4096, H=8, K=64, V=64, seed=SEED_BASE + 7):
    """Matrix associative memory S_t = p (.) S_{t-1} + (1 - p) (.) (v_t (x) k_t),
    p per key: returned as the per-key-scale decay-separable scan (g = log p,
    kappa = 1 - p)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    pk = _sigmoid(rng.standard_normal((B, T, H, K)) + 2.0)
    return dict(q=_bf16(q), k=_bf16(k), v=_bf16(v), g=_f32(np.log(pk)), decay_mode=1,
                k_scale=None, k_scale_key=_f32(1.0 - pk), scale=1.0, s0=None)


def hgrn2(B=4, T=4096, H=16, K=128, V=128, seed=SEED_BASE + 8):
    """HGRN2 shaped scan: GLA's recurrence with the key tied to the per-key
    forget gate, k = 1 - f, decay f."""
    rng = np.random.default_rng(seed)
    f = _sigmoid(rng.standard_normal((B, T, H, K)) + 2.0)
    q = rng.standard_normal((B, T, H, K))
    v = rng.standard_normal((B, T, H, V))
    return dict(q=_bf16(q), k=_bf16(1.0 - f), v=_bf16(v), g=_f32(np.log(f)), decay_mode=1,
                k_scale=None, scale=1.0, s0=None)


def norm_gate_epilogue(B, T, H, V, seed=SEED_BASE + 9):
    """Inputs of GLA's output norm-gate: gate z [B,T,H,V] bf16, RMSNorm weight [V]."""
    rng = np.random.default_rng(seed)
    return dict(gate=_bf16(rng.standard_normal((B, T, H, V))),
                norm_weight=_f32(rng.uniform(0.5, 1.5, size=(V,))), eps=1e-6)


def skip_epilogue(H, seed=SEED_BASE + 10):
    """Mamba-2's per-head skip weight D [H]."""
    rng = np.random.default_rng(seed)
    return dict(d_skip=_f32(rng.uniform(0.5, 1.5, size=(H,))))


def random_state(shape, seed, std=1.0):
    """An fp32 initial state ~ N(0, std^2) for continuation and unit tests."""
    rng = np.random.default_rng(seed)
    return _f32(rng.standard_normal(shape) * std)


def random_normal(shape, seed):
    """An fp32 N(0, 1) tensor of any size, drawn one leading-axis slice at a
    time (incoming gradients, stand-in states of the gradient pass)."""
    rng = np.random.default_rng(seed)
    out = torch.empty(tuple(shape), dtype=torch.float32)
    for i in range(shape[0]):
        out[i] = _f32(rng.standard_normal(tuple(shape[1:])))
    return out


# ---- device-side draws, for tensors past 32-bit offsets ----

def _device_gen(seed, device):
    return torch.Generator(device=device).manual_seed(int(seed))


def _normal_bf16_device(shape, gen, device, unit_rows=False):
    """N(0,1) draws rounded to bf16, one leading-axis slice at a time (so the
    float32 temporaries stay one slice); unit_rows: each last-axis row divided
    by its L2 norm before the rounding."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    for i in range(shape[0]):
        x = torch.randn(shape[1:], generator=gen, device=device)
        if unit_rows:
            x /= x.norm(dim=-1, keepdim=True)
        out[i] = x.to(torch.bfloat16)
    return out


def gated_device(B, T, N, seed=SEED_BASE + 11, device="cuda:0"):
    """The gated recipe on the device: a = sigmoid(z), z ~ N(2,1); u ~ N(0,1);
    s0 ~ N(0,1); fp32 [B,T,N]."""
    gen = _device_gen(seed, device)
    a = torch.randn((B, T, N), generator=gen, device=device).add_(2.0).sigmoid_()
    u = torch.randn((B, T, N), generator=gen, device=device)
    s0 = torch.randn((B, N), generator=gen, device=device)
    return dict(a=a, u=u, s0=s0)


def deltanet_device(B, T, H, K, V, seed=SEED_BASE + 12, device="cuda:0"):
    """The DeltaNet recipe on the device: L2-normalised q, k and v ~ N(0,1) in
    bf16, beta = sigmoid(N(0,1)) fp32."""
    gen = _device_gen(seed, device)
    q = _normal_bf16_device((B, T, H, K), gen, device, unit_rows=True)
    k = _normal_bf16_device((B, T, H, K), gen, device, unit_rows=True)
    v = _normal_bf16_device((B, T, H, V), gen, device)
    beta = torch.randn((B, T, H), generator=gen, device=device).sigmoid_()
    return dict(q=q, k=k, v=v, beta=beta, scale=1.0, s0=None)


def mamba2_device(B, T, H, K, V, seed=SEED_BASE + 13, device="cuda:0"):
    """The Mamba-2 recipe on the device (one B/C group): dt = softplus(N(0,1)),
    A_h = -exp(U(0,2)), g = dt A_h, B, C, x ~ N(0,1) bf16."""
    gen = _device_gen(seed, device)
    dt = torch.nn.functional.softplus(torch.randn((B, T, H), generator=gen, device=device))
    A = -torch.exp(2.0 * torch.rand((H,), generator=gen, device=device))
    g = dt * A
    Bm = _normal_bf16_device((B, T, 1, K), gen, device)
    Cm = _normal_bf16_device((B, T, 1, K), gen, device)
    x = _normal_bf16_device((B, T, H, V), gen, device)
    return dict(q=Cm, k=Bm, v=x, g=g, decay_mode=0, k_scale=dt, scale=1.0, s0=None)


def gla_device(B, T, H, K, V, seed=SEED_BASE + 14, device="cuda:0"):
    """The GLA recipe on the device: q, k, v ~ N(0,1) bf16, per-key
    gk = logsigmoid(N(0,1))/16 fp32, readout scale K**-0.5."""
    gen = _device_gen(seed, device)
    q = _normal_bf16_device((B, T, H, K), gen, device)
    k = _normal_bf16_device((B, T, H, K), gen, device)
    v = _normal_bf16_device((B, T, H, V), gen, device)
    g = torch.empty((B, T, H, K), dtype=torch.float32, device=device)
    for i in range(B):
        g[i] = torch.nn.functional.logsigmoid(torch.randn((T, H, K), generator=gen, device=device)) / 16.0
    return dict(q=q, k=k, v=v, g=g, decay_mode=1, k_scale=None, scale=float(K) ** -0.5, s0=None)


def rwkv7_device(B, T, H, K, V, seed=SEED_BASE + 15, device="cuda:0"):
    """The RWKV-7 recipe on the device: DeltaNet's q, k, v, beta plus the
    per-key log-decay g = -exp(-softplus(-z) - 0.5), z ~ N(0,1), fp32."""
    d = deltanet_device(B, T, H, K, V, seed=seed, device=device)
    gen = _device_gen(seed + 1000, device)
    g = torch.empty((B, T, H, K), dtype=torch.float32, device=device)
    for i in range(B):
        z = torch.randn((T, H, K), generator=gen, device=device)
        g[i] = -torch.exp(-torch.nn.functional.softplus(-z) - 0.5)
    d["g"] = g
    return d


def random_normal_device(shape, seed, device="cuda:0"):
    """An fp32 N(0, 1) tensor drawn on the device (incoming gradients and
    stand-in forward states of the gradient pass at sizes past 32-bit offsets)."""
    return torch.randn(tuple(shape), generator=_device_gen(seed, device), device=device)

