// Delta-rule state scan with readout, on gfx950 matrix cores:
//
//   delta_t = beta_t (v_t - S_{t-1}^T k_t),  S_t = S_{t-1} + k_t delta_t^T,
//   o_t     = scale * S_t^T q_t
//
// [SunnyNet log §4.2: "SunnyNet 工程化实录：一个 O(N) 架构如何长出自己的 C 推理运行时",
//  developer.aliyun.com/article/1773847; restated in "我拿同一份权重和 llama.cpp
//  正面比了一场：我手写的 C 内核，慢了 1.1–1.7 倍" §3].
//
// Chunked (WY / UT) form.  Inside a chunk of L = 64 steps with entering state
// S0, the deltas Delta (L x V) satisfy (I + A) Delta = diag(beta)(V - K S0)
// with A = strict_lower(diag(beta) K K^T), because step t subtracts the
// read-back of the earlier deltas of the same chunk.  So, with
// Tb = (I + A)^{-1} diag(beta):
//   Delta = Tb (V - K S0),   O = scale (Q S0 + tril(Q K^T) Delta),
//   S_L   = S0 + K^T Delta.
// This is the sequential recurrence regrouped exactly (the pages call the
// rank-1 form token-serial; the regrouping changes only the order of
// additions).
//
// Two kernels:
//  * delta_prep: one workgroup per (batch, head, chunk), all in parallel.  It
//    forms A on the matrix cores (bf16 keys enter exactly), inverts I + A by
//    blocked forward substitution in fp32 (16 x 16 diagonal blocks, then the
//    off-diagonal blocks in three dependent stages), and stores Tb as a pair of
//    bf16 planes (hi + lo ~ fp32) in the context workspace.
//  * delta_scan: one workgroup per (batch, head, V-tile of VT columns) walks the
//    chunks in order with its K x VT state tile in registers, prefetching the
//    next chunk (q, k, v tile, Tb) while computing the current one.  Per chunk:
//    M = tril(Q K^T) and Y = K S0 (matrix cores), R = V - Y, Delta = Tb R,
//    O = scale (Q S0 + M Delta), S += K^T Delta.  fp32 operands of the matrix
//    cores are split into hi + lo bf16 terms.
//  Arrays that must be stored transposed in LDS (K^T for the state update) are
//  loaded with lanes running along time, so the transposed 2-byte LDS writes of
//  a wave land in consecutive halfwords (no bank conflicts).
#include "lrs_internal.h"
#include "mfma_util.h"

namespace lrs {
namespace {

constexpr int L = 64;
constexpr int NT = 256;

struct DeltaArgs {
    const u16* q;
    const u16* k;
    const u16* v;
    const float* beta;
    const float* s0;
    float* o;
    float* s_final;
    u16* tb;          // workspace: per (b,h,chunk) two 64x64 bf16 planes (hi, lo)
    int B, T, H, K, V;
    float scale;
    int vtiles;
    int nchunks;
};

__device__ __forceinline__ void tri_block(int n, int& i, int& j) {
    i = n < 1 ? 0 : (n < 3 ? 1 : (n < 6 ? 2 : 3));
    j = n - (i * (i + 1)) / 2;
}

// 8-byte LDS write of 4 bf16.
__device__ __forceinline__ void store4(u16* dst, u16 a, u16 b, u16 c, u16 d) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    u32x2 w = {a | (static_cast<uint32_t>(b) << 16), c | (static_cast<uint32_t>(d) << 16)};
    *reinterpret_cast<u32x2*>(dst) = w;
}

// ---------------------------------------------------------------------------
// prep: Tb = (I + strict_lower(diag(beta) K K^T))^{-1} diag(beta) per chunk
// ---------------------------------------------------------------------------
template <int KP, bool VEC>
__global__ __launch_bounds__(NT) void delta_prep_kernel(DeltaArgs p) {
    constexpr int LDK = KP + 8;
    constexpr int LDA = L + 1;   // fp32 rows, odd stride
    __shared__ __align__(16) u16 sK[L * LDK];
    __shared__ float sA[L * LDA];
    __shared__ float sT[L * LDA];
    __shared__ float sY[16 * L];
    __shared__ float sBeta[L];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = blockIdx.x % p.nchunks;
    const int bh = blockIdx.x / p.nchunks;
    const int b = bh / p.H, h = bh - b * p.H;
    const int64_t T = p.T, t0 = static_cast<int64_t>(c) * L;
    const int K = p.K;

    const BufRes rk = make_rsrc(p.k + b * T * p.H * static_cast<int64_t>(K), T * p.H * static_cast<int64_t>(K) * 2);
    for (int pi = tid; pi < L * KP / 8; pi += NT) {
        const int row = pi / (KP / 8), c8 = (pi % (KP / 8)) * 8;
        const int64_t t = t0 + row;
        u32x4 x = {0u, 0u, 0u, 0u};
        if constexpr (VEC) {
            x = buf_load16(rk, c8 < K ? ((static_cast<int>(t) * p.H + h) * K + c8) * 2 : kBufOOB);
        } else {
            if (t < T) x = load8_bf16(p.k + ((b * T + t) * p.H + h) * static_cast<int64_t>(K), c8, K, false);
        }
        *reinterpret_cast<u32x4*>(sK + row * LDK + c8) = x;
    }
    if (tid < L) sBeta[tid] = (t0 + tid < T) ? p.beta[(b * T + t0 + tid) * p.H + h] : 0.0f;
    for (int e = tid; e < L * LDA; e += NT) {
        sA[e] = 0.0f;
        sT[e] = 0.0f;
    }
    __syncthreads();

    // A = strict_lower(diag(beta) K K^T): keys are bf16, products exact in fp32
    for (int n = wave; n < 10; n += 4) {
        int bi, bj;
        tri_block(n, bi, bj);
        f32x4 acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < KP; k0 += 32)
            acc = mfma16(frag<LDK>(sK, 16 * bi, k0, lane), frag<LDK>(sK, 16 * bj, k0, lane), acc);
        const int tau = 16 * bj + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * bi + 4 * (lane >> 4) + r;
            if (tau < t) sA[t * LDA + tau] = sBeta[t] * acc[r];
        }
    }
    __syncthreads();

    // diagonal 16x16 blocks of (I + A)^{-1}: forward substitution, one lane per column
    if (tid < L) {
        const int bk = tid / 16, col = tid % 16;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = (i == col) ? 1.0f : 0.0f;
#pragma unroll
            for (int j = 0; j < i; ++j) s -= sA[(16 * bk + i) * LDA + 16 * bk + j] * x[j];
            x[i] = s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[(16 * bk + i) * LDA + 16 * bk + col] = x[i];
    }
    __syncthreads();

    // off-diagonal blocks, block row by block row:
    //   T[i][col] = T_ii * ( - sum_{m=j..i-1} A_im T_m[col] ),  col in block j < i
    for (int bi = 1; bi < 4; ++bi) {
        const int col = tid % L, qr = tid / L;   // qr: which 4 rows of the block
        const bool act = col < 16 * bi;
        if (act) {
            const int bj = col / 16;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = 4 * qr + rr;
                float y = 0.0f;
                for (int m = 16 * bj; m < 16 * bi; ++m) y -= sA[(16 * bi + r) * LDA + m] * sT[m * LDA + col];
                sY[r * L + col] = y;
            }
        }
        __syncthreads();
        if (act) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = 4 * qr + rr;
                float x = 0.0f;
#pragma unroll
                for (int s2 = 0; s2 < 16; ++s2) x += sT[(16 * bi + r) * LDA + 16 * bi + s2] * sY[s2 * L + col];
                sT[(16 * bi + r) * LDA + col] = x;
            }
        }
        __syncthreads();
    }

    // Tb = T diag(beta) as hi/lo bf16 planes, row-major 64 x 64
    u16* dst = p.tb + static_cast<int64_t>(blockIdx.x) * 2 * L * L;
    {
        const int row = tid / 4, c0 = (tid % 4) * 16;
        u16 hi[16], lo[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) split_bf16(sT[row * LDA + c0 + e] * sBeta[c0 + e], hi[e], lo[e]);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            u32x4 wh, wl;
            wh.x = hi[8 * half + 0] | (static_cast<uint32_t>(hi[8 * half + 1]) << 16);
            wh.y = hi[8 * half + 2] | (static_cast<uint32_t>(hi[8 * half + 3]) << 16);
            wh.z = hi[8 * half + 4] | (static_cast<uint32_t>(hi[8 * half + 5]) << 16);
            wh.w = hi[8 * half + 6] | (static_cast<uint32_t>(hi[8 * half + 7]) << 16);
            wl.x = lo[8 * half + 0] | (static_cast<uint32_t>(lo[8 * half + 1]) << 16);
            wl.y = lo[8 * half + 2] | (static_cast<uint32_t>(lo[8 * half + 3]) << 16);
            wl.z = lo[8 * half + 4] | (static_cast<uint32_t>(lo[8 * half + 5]) << 16);
            wl.w = lo[8 * half + 6] | (static_cast<uint32_t>(lo[8 * half + 7]) << 16);
            *reinterpret_cast<u32x4*>(dst + row * L + c0 + 8 * half) = wh;
            *reinterpret_cast<u32x4*>(dst + L * L + row * L + c0 + 8 * half) = wl;
        }
    }
}

// ---------------------------------------------------------------------------
// scan: sequential over chunks per (batch, head, V-tile)
// ---------------------------------------------------------------------------
template <int KP, int VT, bool VEC>
__global__ __launch_bounds__(NT) void delta_scan_kernel(DeltaArgs p) {
    constexpr int LDK = KP + 8;
    constexpr int LDL = L + 8;
    constexpr int LDV = VT + 8;
    constexpr int KT = KP / 16;
    constexpr int VTT = VT / 16;
    constexpr int S_PER_WAVE = KT * VTT / 4;
    constexpr int PQ = L * KP / 8 / NT;        // q/k pieces per thread
    constexpr int NVP = L * VT / 8;            // v pieces per chunk
    constexpr int PVT = (NVP + NT - 1) / NT;   // v pieces per thread
    constexpr int PT = 2 * L * L / 8 / NT;     // Tb pieces per thread (hi + lo)
    static_assert(PQ >= 1 && S_PER_WAVE >= 1, "tile shape");

    __shared__ __align__(16) u16 sQ[L * LDK];
    __shared__ __align__(16) u16 sK[L * LDK];
    __shared__ __align__(16) u16 sKT[KP * LDL];
    __shared__ __align__(16) u16 sTh[L * LDL];
    __shared__ __align__(16) u16 sTl[L * LDL];
    __shared__ __align__(16) u16 sMh[L * LDL];
    __shared__ __align__(16) u16 sMl[L * LDL];
    __shared__ __align__(16) u16 sV[L * LDV];
    __shared__ __align__(16) u16 sRTh[VT * LDL];
    __shared__ __align__(16) u16 sRTl[VT * LDL];
    __shared__ __align__(16) u16 sDTh[VT * LDL];
    __shared__ __align__(16) u16 sDTl[VT * LDL];
    __shared__ __align__(16) u16 sSTh[VT * LDK];
    __shared__ __align__(16) u16 sSTl[VT * LDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
    const int vt = lid % p.vtiles;
    const int bh = lid / p.vtiles;
    const int b = bh / p.H, h = bh - b * p.H;
    const int v0 = vt * VT;
    const int64_t T = p.T;
    const int K = p.K, V = p.V, H = p.H;
    const int nchunks = p.nchunks;
    const u16* tbase = p.tb + static_cast<int64_t>(bh) * nchunks * 2 * L * L;

    // q/k pieces: row = pi % 64 (lanes along time), columns c8 = 8 * (pi / 64).
    // Vector path: per-batch-row buffer resources; rows past T and columns past
    // K / V read as zero in hardware, so the prefetch is a straight run of loads.
    const int64_t qk_row = static_cast<int64_t>(H) * K, v_row = static_cast<int64_t>(H) * V;
    const BufRes rq = make_rsrc(p.q + b * T * qk_row, T * qk_row * 2);
    const BufRes rk = make_rsrc(p.k + b * T * qk_row, T * qk_row * 2);
    const BufRes rv = make_rsrc(p.v + b * T * v_row, T * v_row * 2);
    const BufRes rt = make_rsrc(tbase, static_cast<int64_t>(nchunks) * 2 * L * L * 2);
    u32x4 cq[PQ], ck[PQ], nq[PQ], nk[PQ], cv[PVT], nv[PVT], ct[PT], nt[PT];
    auto load_chunk = [&](int c, u32x4 (&Q)[PQ], u32x4 (&Kx)[PQ], u32x4 (&Vx)[PVT], u32x4 (&Tx)[PT]) {
        const int64_t t0 = static_cast<int64_t>(c) * L;
        if constexpr (VEC) {
#pragma unroll
            for (int i = 0; i < PQ; ++i) {
                const int pi = tid + NT * i;
                const int row = pi % L, c8 = (pi / L) * 8;
                const int t = static_cast<int>(t0) + row;
                const int off = c8 < K ? ((t * H + h) * K + c8) * 2 : kBufOOB;
                Q[i] = buf_load16(rq, off);
                Kx[i] = buf_load16(rk, off);
            }
#pragma unroll
            for (int i = 0; i < PVT; ++i) {
                const int pi = tid + NT * i;
                const int row = pi % L, c8 = (pi / L) * 8;
                const int t = static_cast<int>(t0) + row;
                const int off = (pi < NVP && v0 + c8 < V) ? ((t * H + h) * V + v0 + c8) * 2 : kBufOOB;
                Vx[i] = buf_load16(rv, off);
            }
        } else {
#pragma unroll
            for (int i = 0; i < PQ; ++i) {
                const int pi = tid + NT * i;
                const int row = pi % L, c8 = (pi / L) * 8;
                const int64_t t = t0 + row;
                Q[i] = u32x4{0u, 0u, 0u, 0u};
                Kx[i] = u32x4{0u, 0u, 0u, 0u};
                if (t < T) {
                    const int64_t off = ((b * T + t) * H + h) * static_cast<int64_t>(K);
                    Q[i] = load8_bf16(p.q + off, c8, K, false);
                    Kx[i] = load8_bf16(p.k + off, c8, K, false);
                }
            }
#pragma unroll
            for (int i = 0; i < PVT; ++i) {
                const int pi = tid + NT * i;
                Vx[i] = u32x4{0u, 0u, 0u, 0u};
                if (pi < NVP) {
                    const int row = pi % L, c8 = (pi / L) * 8;
                    const int64_t t = t0 + row;
                    if (t < T)
                        Vx[i] = load8_bf16(p.v + ((b * T + t) * H + h) * static_cast<int64_t>(V) + v0, c8,
                                           V - v0, false);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int pi = tid + NT * i;   // hi plane pieces 0..511, lo plane 512..1023
            Tx[i] = buf_load16(rt, (c * 2 * L * L + 8 * pi) * 2);
        }
    };

    // state tile from s0
    f32x4 S[S_PER_WAVE];
#pragma unroll
    for (int m = 0; m < S_PER_WAVE; ++m) {
        const int s = wave * S_PER_WAVE + m, sr = s / VTT, sc = s % VTT;
        const int j = v0 + 16 * sc + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = 16 * sr + 4 * (lane >> 4) + r;
            float x = 0.0f;
            if (p.s0 && d < K && j < V) x = p.s0[((static_cast<int64_t>(b) * H + h) * K + d) * V + j];
            S[m][r] = x;
        }
    }
    auto write_state_lds = [&]() {
#pragma unroll
        for (int m = 0; m < S_PER_WAVE; ++m) {
            const int s = wave * S_PER_WAVE + m, sr = s / VTT, sc = s % VTT;
            const int j = 16 * sc + (lane & 15);
            const int d = 16 * sr + 4 * (lane >> 4);
            u16 hi[4], lo[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) split_bf16(S[m][r], hi[r], lo[r]);
            store4(sSTh + j * LDK + d, hi[0], hi[1], hi[2], hi[3]);
            store4(sSTl + j * LDK + d, lo[0], lo[1], lo[2], lo[3]);
        }
    };
    write_state_lds();
    // blocks of M above the diagonal are never written and must read as zero
    for (int e = tid; e < L * LDL; e += NT) {
        sMh[e] = 0;
        sMl[e] = 0;
    }
    load_chunk(0, cq, ck, cv, ct);

    for (int c = 0; c < nchunks; ++c) {
        const int64_t t0 = static_cast<int64_t>(c) * L;
        // ---- P0: chunk inputs into LDS ----
#pragma unroll
        for (int i = 0; i < PQ; ++i) {
            const int pi = tid + NT * i;
            const int row = pi % L, c8 = (pi / L) * 8;
            *reinterpret_cast<u32x4*>(sQ + row * LDK + c8) = cq[i];
            *reinterpret_cast<u32x4*>(sK + row * LDK + c8) = ck[i];
#pragma unroll
            for (int e = 0; e < 8; ++e) sKT[(c8 + e) * LDL + row] = piece_elem(ck[i], e);
        }
#pragma unroll
        for (int i = 0; i < PVT; ++i) {
            const int pi = tid + NT * i;
            if (pi < NVP) {
                const int row = pi % L, c8 = (pi / L) * 8;
                *reinterpret_cast<u32x4*>(sV + row * LDV + c8) = cv[i];
            }
        }
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int pi = tid + NT * i;
            const int plane = pi / (L * L / 8), pp = pi % (L * L / 8);
            const int row = pp / (L / 8), c8 = (pp % (L / 8)) * 8;
            *reinterpret_cast<u32x4*>((plane ? sTl : sTh) + row * LDL + c8) = ct[i];
        }
        __syncthreads();
        if (c + 1 < nchunks) load_chunk(c + 1, nq, nk, nv, nt);

        // ---- P1: M = tril(Q K^T) (exact), Y = K S0 -> R = V - Y, O1 = Q S0 ----
        for (int n = wave; n < 10; n += 4) {
            int bi, bj;
            tri_block(n, bi, bj);
            f32x4 acc = zero4();
#pragma unroll
            for (int k0 = 0; k0 < KP; k0 += 32)
                acc = mfma16(frag<LDK>(sQ, 16 * bi, k0, lane), frag<LDK>(sK, 16 * bj, k0, lane), acc);
            const int tau = 16 * bj + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * bi + 4 * (lane >> 4) + r;
                u16 hi, lo;
                split_bf16(tau <= t ? acc[r] : 0.0f, hi, lo);
                sMh[t * LDL + tau] = hi;
                sMl[t * LDL + tau] = lo;
            }
        }
        const int ri = wave;
        f32x4 O1[VTT];
#pragma unroll
        for (int cj = 0; cj < VTT; ++cj) {
            f32x4 y = zero4(), o1 = zero4();
#pragma unroll
            for (int k0 = 0; k0 < KP; k0 += 32) {
                const bf16x8 sh = frag<LDK>(sSTh, 16 * cj, k0, lane);
                const bf16x8 sl = frag<LDK>(sSTl, 16 * cj, k0, lane);
                const bf16x8 ka = frag<LDK>(sK, 16 * ri, k0, lane);
                const bf16x8 qa = frag<LDK>(sQ, 16 * ri, k0, lane);
                y = mfma16(ka, sl, y);
                y = mfma16(ka, sh, y);
                o1 = mfma16(qa, sl, o1);
                o1 = mfma16(qa, sh, o1);
            }
            O1[cj] = o1;
            const int j = 16 * cj + (lane & 15);
            const int t = 16 * ri + 4 * (lane >> 4);
            u16 hi[4], lo[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) split_bf16(bf2f(sV[(t + r) * LDV + j]) - y[r], hi[r], lo[r]);
            store4(sRTh + j * LDL + t, hi[0], hi[1], hi[2], hi[3]);
            store4(sRTl + j * LDL + t, lo[0], lo[1], lo[2], lo[3]);
        }
        __syncthreads();

        // ---- P2: Delta = Tb R (row block = wave) ----
#pragma unroll
        for (int cj = 0; cj < VTT; ++cj) {
            f32x4 dl = zero4();
            for (int ks = 0; ks <= ri / 2; ++ks) {
                const bf16x8 th = frag<LDL>(sTh, 16 * ri, 32 * ks, lane);
                const bf16x8 tl = frag<LDL>(sTl, 16 * ri, 32 * ks, lane);
                const bf16x8 rh = frag<LDL>(sRTh, 16 * cj, 32 * ks, lane);
                const bf16x8 rl = frag<LDL>(sRTl, 16 * cj, 32 * ks, lane);
                dl = mfma16(tl, rh, dl);
                dl = mfma16(th, rl, dl);
                dl = mfma16(th, rh, dl);
            }
            const int j = 16 * cj + (lane & 15);
            const int t = 16 * ri + 4 * (lane >> 4);
            u16 hi[4], lo[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) split_bf16(dl[r], hi[r], lo[r]);
            store4(sDTh + j * LDL + t, hi[0], hi[1], hi[2], hi[3]);
            store4(sDTl + j * LDL + t, lo[0], lo[1], lo[2], lo[3]);
        }
        __syncthreads();

        // ---- P3: O = scale (O1 + M Delta); S += K^T Delta ----
#pragma unroll
        for (int cj = 0; cj < VTT; ++cj) {
            f32x4 o2 = zero4();
            for (int ks = 0; ks <= ri / 2; ++ks) {
                const bf16x8 mh = frag<LDL>(sMh, 16 * ri, 32 * ks, lane);
                const bf16x8 ml = frag<LDL>(sMl, 16 * ri, 32 * ks, lane);
                const bf16x8 dh = frag<LDL>(sDTh, 16 * cj, 32 * ks, lane);
                const bf16x8 dlo = frag<LDL>(sDTl, 16 * cj, 32 * ks, lane);
                o2 = mfma16(ml, dh, o2);
                o2 = mfma16(mh, dlo, o2);
                o2 = mfma16(mh, dh, o2);
            }
            const int j = v0 + 16 * cj + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * ri + 4 * (lane >> 4) + r;
                if (t0 + t < T && j < V)
                    p.o[((b * T + t0 + t) * H + h) * static_cast<int64_t>(V) + j] = p.scale * (O1[cj][r] + o2[r]);
            }
        }
#pragma unroll
        for (int m = 0; m < S_PER_WAVE; ++m) {
            const int s = wave * S_PER_WAVE + m, sr = s / VTT, sc = s % VTT;
            f32x4 ds = zero4();
#pragma unroll
            for (int ks = 0; ks < L / 32; ++ks) {
                const bf16x8 ka = frag<LDL>(sKT, 16 * sr, 32 * ks, lane);
                ds = mfma16(ka, frag<LDL>(sDTl, 16 * sc, 32 * ks, lane), ds);
                ds = mfma16(ka, frag<LDL>(sDTh, 16 * sc, 32 * ks, lane), ds);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) S[m][r] += ds[r];
        }
        __syncthreads();
        write_state_lds();

        if (c + 1 < nchunks) {
#pragma unroll
            for (int i = 0; i < PQ; ++i) { cq[i] = nq[i]; ck[i] = nk[i]; }
#pragma unroll
            for (int i = 0; i < PVT; ++i) cv[i] = nv[i];
#pragma unroll
            for (int i = 0; i < PT; ++i) ct[i] = nt[i];
        }
    }

#pragma unroll
    for (int m = 0; m < S_PER_WAVE; ++m) {
        const int s = wave * S_PER_WAVE + m, sr = s / VTT, sc = s % VTT;
        const int j = v0 + 16 * sc + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = 16 * sr + 4 * (lane >> 4) + r;
            if (d < K && j < V) p.s_final[((static_cast<int64_t>(b) * H + h) * K + d) * V + j] = S[m][r];
        }
    }
}

template <int KP, int VT>
hipError_t launch_t(const DeltaArgs& a, bool vec, hipStream_t stream) {
    const int64_t gprep = static_cast<int64_t>(a.B) * a.H * a.nchunks;
    const int64_t gscan = static_cast<int64_t>(a.B) * a.H * a.vtiles;
    if (vec) {
        hipLaunchKernelGGL((delta_prep_kernel<KP, true>), dim3(static_cast<unsigned>(gprep)), dim3(NT), 0,
                           stream, a);
        hipLaunchKernelGGL((delta_scan_kernel<KP, VT, true>), dim3(static_cast<unsigned>(gscan)), dim3(NT), 0,
                           stream, a);
    } else {
        hipLaunchKernelGGL((delta_prep_kernel<KP, false>), dim3(static_cast<unsigned>(gprep)), dim3(NT), 0,
                           stream, a);
        hipLaunchKernelGGL((delta_scan_kernel<KP, VT, false>), dim3(static_cast<unsigned>(gscan)), dim3(NT), 0,
                           stream, a);
    }
    return hipGetLastError();
}

}  // namespace

int delta_vtile() { return 16; }

size_t delta_workspace_bytes(int B, int T, int H) {
    const int64_t nchunks = (static_cast<int64_t>(T) + L - 1) / L;
    return static_cast<size_t>(B) * H * nchunks * 2 * L * L * sizeof(u16);
}

hipError_t launch_scan_delta(const DeltaParams& prm, void* workspace, hipStream_t stream) {
    DeltaArgs a{};
    a.q = reinterpret_cast<const u16*>(prm.q);
    a.k = reinterpret_cast<const u16*>(prm.k);
    a.v = reinterpret_cast<const u16*>(prm.v);
    a.beta = prm.beta;
    a.s0 = prm.s0;
    a.o = prm.o;
    a.s_final = prm.s_final;
    a.tb = static_cast<u16*>(workspace);
    a.B = prm.B;
    a.T = prm.T;
    a.H = prm.H;
    a.K = prm.K;
    a.V = prm.V;
    a.scale = prm.scale;
    a.vtiles = (prm.V + delta_vtile() - 1) / delta_vtile();
    a.nchunks = (prm.T + L - 1) / L;
    return prm.K <= 64 ? launch_t<64, 16>(a, prm.vec != 0, stream) : launch_t<128, 16>(a, prm.vec != 0, stream);
}

}  // namespace lrs
