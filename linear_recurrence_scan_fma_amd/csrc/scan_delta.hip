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
// read-back of the earlier deltas of the same chunk.  With
// Tb = (I + A)^{-1} diag(beta), MTb = tril(Q K^T) Tb and W = K^T Tb:
//   R = V - K S0,   O = scale (Q S0 + MTb R),   S_L = S0 + W R
// (Delta = Tb R itself is never formed).  This is the sequential recurrence
// regrouped exactly (the pages call the rank-1 form token-serial; the
// regrouping changes only the order of additions).
//
// With a per-key decay (RWKV-7's update [SunnyNet log §5.1], read key-major):
//   delta_t = beta_t (v_t - S_{t-1}^T k_t),  S_t = diag(w_t) S_{t-1} + k_t delta_t^T,
// w_t = exp(g_t).  With G_t the running sum of g inside the chunk (G_{-1} = 0),
// unrolling the chunk gives the same form on decayed operands (per key):
//   a_t = e^{G_{t-1}} k_t,  b_t = e^{-G_t} k_t,  qt_t = e^{G_t} q_t,  khat_t = e^{G_L - G_t} k_t,
//   A = strict_lower(diag(beta) a b^T),  MTb = tril(qt b^T) Tb,  W = khat^T Tb,
//   R = V - a S0,  O = scale (qt S0 + MTb R),  S_L = diag(e^{G_L}) S0 + W R.
//
// Two kernels:
//  * delta_prep, one workgroup per (batch, head, chunk), all in parallel:
//    A and tril(Q K^T) on the matrix cores; the 16x16 diagonal blocks of
//    (I + A)^{-1} by forward substitution, the off-diagonal blocks column
//    block by column block, each in one wave with no barrier, on 16x16x16
//    matrix-core products whose 16x16 result is laid out exactly as the next
//    product's right operand; then MTb and W, stored as hi/lo bf16 planes
//    (hi + lo ~ fp32).  The decayed form takes the running log-decay per key,
//    forms a b^T and qt b^T from hi/lo operands scaled about the chunk's
//    middle step (every factor within e^{+-30} while no key's running sum
//    strays more than 30 nats from its middle value; past that it takes the
//    pairs one by one with exact exponentials), and also stores a and qt as
//    hi/lo planes and e^{G_L}, so the scan does no transcendental work.
//  * delta_scan, one workgroup per (batch, head, 16-wide V-tile), walks the
//    chunks in order with its K x 16 state in registers.  Per chunk, two
//    phases and two barriers: Y = K S0 (a S0) and Q S0 (qt S0), R = V - Y;
//    then MTb R for the outputs and S = S0 + W R (diag(e^{G_L}) S0 + W R).
//    fp32 operands are split into hi + lo bf16 terms.  K <= 128 in both forms.
//
// Time segments, where the (batch, head, V-tile) workgroups would leave most
// of the device idle: a chunk maps its entering state affinely,
// S_L = (I - W K) S0 + W V (decayed: (diag(e^{G_L}) - W a) S0 + W V), so a
// run of chunks does too, S_out = A_s S_in + B_s.  A segment pass (the scan
// without its readout) runs segment 0 from s0 and, for every later segment
// but the last, K identity columns with zero values (their state at the end
// is A_s) beside state columns from zero (B_s); delta_seg_prefix chains the
// entering states in fp32; then the scan runs every segment at once from its
// entering state.
#include "lrs_internal.h"
#include "mfma_util.h"

namespace lrs {
namespace {

constexpr int L = 64;
constexpr int NT = 256;
constexpr int PLANE = L * L;   // elements of one 64 x 64 bf16 plane
constexpr int VT = 16;         // V-tile width of the scan kernel
constexpr int KD = 128;        // largest key width of the decayed form
constexpr float kHalfSpan = 30.0f;   // decayed prep: factor exponents stay within +-30 nats

// One chunk's workspace block, in u16 elements:
//   MTb hi, MTb lo          4 x 2 x 2 blocks of 512: MTb in the scan's operand
//                           order (as W; blocks above the diagonal unused)
//   W hi, W lo              KP / 16 x 2 x 2 blocks of 512: W in the scan's
//                           operand order (below)
//   decayed form only:
//   a hi, a lo, qt hi, qt lo   4 x [L][KP]
//   e^{G_L}                    [KP] fp32
template <int KP>
constexpr int off_w() { return 2 * PLANE; }
// W (KP keys x 64 steps) is stored as the scan's 16x16x32 operand fragments:
// block (key tile kt, step half ks, hi/lo hl) of 512 elements holds, for
// lane l, keys 16 kt + l % 16 and steps 32 ks + 8 (l / 16) .. +7, so that each
// of the scan's loads reads one contiguous kilobyte (whole cache lines).
__device__ __forceinline__ int wfrag_off(int kt, int ks, int hl) { return ((kt * 2 + ks) * 2 + hl) * 512; }
// MTb (64 steps t x 64 steps tau) in the same order: block (row tile rb, step
// half ks, hi/lo) holds, for lane l, rows 16 rb + l % 16 and columns
// 32 ks + 8 (l / 16) .. +7.  The scan reads blocks with ks <= rb / 2 only.
__device__ __forceinline__ int mfrag_off(int rb, int ks, int hl) { return ((rb * 2 + ks) * 2 + hl) * 512; }
template <int KP>
constexpr int off_aq() { return 2 * PLANE + 2 * KP * L; }
template <int KP>
constexpr int off_el() { return off_aq<KP>() + 4 * L * KP; }
template <int KP, bool DECAY>
constexpr int chunk_u16() {
    return DECAY ? off_el<KP>() + 2 * KP : off_aq<KP>();
}


struct DeltaArgs {
    const u16* q;
    const u16* k;
    const u16* v;
    const float* beta;
    const float* g;   // per-key log-decay [B,T,H,K] (decayed form only)
    const float* s0;
    float* o;
    float* s_final;
    u16* ws;          // per (b,h,chunk): one chunk_u16() block
    int B, T, H, K, V;
    float scale;
    int vtiles;
    int nchunks;
    int out_bf16;     // o is bf16 (round to nearest even) instead of fp32
    // time segments (nseg = 1: one pass over all chunks).  Segment s covers
    // chunks [s cps, (s + 1) cps); across a segment the state obeys
    // S_out = A_s S_in + B_s.  seg_state[s] ([B][H][K][V] fp32) is the state
    // entering segment s (s >= 1); seg_ab[s] ([B][H][K][K + V] fp32) holds A_s
    // in its first K columns and B_s after them (1 <= s <= nseg - 2).
    int nseg, cps;
    float* seg_state;
    float* seg_ab;
};

__device__ __forceinline__ void tri_block(int n, int& i, int& j) {
    i = n < 1 ? 0 : (n < 3 ? 1 : (n < 6 ? 2 : 3));
    j = n - (i * (i + 1)) / 2;
}

// MTb output blocks (i, j) handled by each wave, five 16x16 block products per
// wave: {(3,0),(0,0)}, {(2,0),(1,0)}, {(3,1),(2,1)}, {(3,2),(1,1),(2,2),(3,3)}.
__device__ __forceinline__ void mtb_job(int wave, int q, int& i, int& j) {
    i = -1;
    j = -1;
    switch (wave * 4 + q) {
        case 0: i = 3; j = 0; break;
        case 1: i = 0; j = 0; break;
        case 4: i = 2; j = 0; break;
        case 5: i = 1; j = 0; break;
        case 8: i = 3; j = 1; break;
        case 9: i = 2; j = 1; break;
        case 12: i = 3; j = 2; break;
        case 13: i = 1; j = 1; break;
        case 14: i = 2; j = 2; break;
        case 15: i = 3; j = 3; break;
        default: break;
    }
}

__device__ __forceinline__ void store4(u16* dst, u16 a, u16 b, u16 c, u16 d) {
    u32x2 w = {a | (static_cast<uint32_t>(b) << 16), c | (static_cast<uint32_t>(d) << 16)};
    *reinterpret_cast<u32x2*>(dst) = w;
}

__device__ __forceinline__ f32x4 mfma16k16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split4(f32x4 x, s16x4& hi, s16x4& lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        u16 hh, ll;
        split_bf16(x[e], hh, ll);
        hi[e] = static_cast<short>(hh);
        lo[e] = static_cast<short>(ll);
    }
}

// acc += X * Y for 16 x 16 fp32 blocks with ~fp32 accuracy.  `xa` is X as the
// left operand of v_mfma_f32_16x16x16_bf16 (lane: row lane%16, k = 4(lane/16)+e)
// and `yb` is Y as the right operand (lane: column lane%16, same k) -- which is
// also how a 16x16 result is laid out, so results chain without a shuffle.
__device__ __forceinline__ f32x4 mm16(f32x4 xa, f32x4 yb, f32x4 acc) {
    s16x4 ah, al, bh, bl;
    split4(xa, ah, al);
    split4(yb, bh, bl);
    acc = mfma16k16(al, bh, acc);
    acc = mfma16k16(ah, bl, acc);
    return mfma16k16(ah, bh, acc);
}

// As mm16 with the right operand already split into hi/lo.
__device__ __forceinline__ f32x4 mm16_rb(f32x4 xa, s16x4 bh, s16x4 bl, f32x4 acc) {
    s16x4 ah, al;
    split4(xa, ah, al);
    acc = mfma16k16(al, bh, acc);
    acc = mfma16k16(ah, bl, acc);
    return mfma16k16(ah, bh, acc);
}

// As mm16 with the left operand already split into hi/lo.
__device__ __forceinline__ f32x4 mm16_la(s16x4 ah, s16x4 al, f32x4 yb, f32x4 acc) {
    s16x4 bh, bl;
    split4(yb, bh, bl);
    acc = mfma16k16(al, bh, acc);
    acc = mfma16k16(ah, bl, acc);
    return mfma16k16(ah, bh, acc);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// 8 consecutive bf16 (columns c0..c0+7 of a row of n columns); zero past the
// row count or past n.  Vector path: one buffer load at `off_bytes` within a
// per-batch-row resource.  Scalar path: from `rowptr`.
template <bool VEC>
__device__ __forceinline__ u32x4 load_piece(BufRes r, const u16* rowptr, int off_bytes, int c0, int n,
                                            bool row_ok) {
    if constexpr (VEC) {
        return buf_load16(r, c0 < n ? off_bytes : kBufOOB);
    } else {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row_ok) x = load8_bf16(rowptr, c0, n, false);
        return x;
    }
}

// ---------------------------------------------------------------------------
// prep: Tb = (I + strict_lower(diag(beta) K K^T))^{-1} diag(beta), MTb = tril(Q K^T) Tb
// ---------------------------------------------------------------------------
// Decayed-form prep tiles: [L][KP] bf16, unpadded, 16-byte piece p of row r
// stored at piece p ^ (r mod KP / 8), so the rows of a 16-byte fragment read
// fall on distinct banks.  Element offset of (row, column):
template <int KP>
__device__ __forceinline__ int tswz(int r, int i) {
    return r * KP + ((((i >> 3) ^ (r & (KP / 8 - 1)))) << 3) + (i & 7);
}

// 16x16x32 operand fragment (rows r0.., columns k0 + 8 (lane / 16) ..) of such a tile
template <int KP>
__device__ __forceinline__ bf16x8 tfrag(const u16* t, int r0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8*>(t + tswz<KP>(r0 + (lane & 15), k0 + 8 * (lane >> 4)));
}

template <int KP, bool VEC, bool DECAY>
__global__ __launch_bounds__(NT) void delta_prep_kernel(DeltaArgs p) {
    static_assert(!DECAY || KP == 64 || KP == KD, "decayed form: K <= 128");
    constexpr int LDK = KP + 8;
    constexpr int LDA = L + 4;                     // fp32 rows of 272 bytes
    constexpr int LDG = KP + 4;                    // fp32 rows of the running log-decay G
    // plain form: sQ, sK as padded rows.  Decayed form: four unpadded tiles
    // whose 16-byte pieces are rotated by an XOR of the row (a hi/lo, later
    // overwritten by qt hi/lo, and b hi/lo), then the running log-decay G; the
    // whole block is dead once A and M are formed, so sA and sT reuse it.  At
    // K = 128 the tiles hold half the keys and A and M are summed over the two
    // halves in turn, so two workgroups fit a compute unit instead of one (prep
    // ~171 -> ~120 us at B=4 T=4096 H=8); at K = 64 the registers, not the LDS,
    // hold it to three workgroups, and the halves' extra barriers only cost.
    constexpr int KH = KP > 64 ? KP / 2 : KP;      // keys per tile
    constexpr int NHALF = KP / KH;
    constexpr int TILE_D = L * KH * 2;
    constexpr int G_OFF = 4 * TILE_D;
    constexpr int QK_BYTES = DECAY ? G_OFF + L * LDG * 4 : 2 * L * LDK * 2;
    constexpr int AT_BYTES = 2 * L * LDA * 4;      // sA, sT (fp32) reuse the same space
    // khat for W ([L][KP] bf16, hi and lo in the decayed form) goes into M's
    // space, or past sA and sT where it does not fit there (decayed, K = 128)
    constexpr int KHAT_BYTES = (DECAY ? 2 : 1) * L * KP * 2;
    constexpr bool KH_PAST = KHAT_BYTES > L * LDA * 4;
    constexpr int AK_BYTES = AT_BYTES + (KH_PAST ? KHAT_BYTES : 0);
    constexpr int U_BYTES = QK_BYTES > AK_BYTES ? QK_BYTES : AK_BYTES;
    __shared__ __align__(16) unsigned char sU[U_BYTES];
    __shared__ __align__(16) float sBeta[L];
    __shared__ float sTot[DECAY ? 4 : 1][DECAY ? KP : 1];
    __shared__ float sRef[DECAY ? KP : 1];
    u16* tile = reinterpret_cast<u16*>(sU);
    u16* sQ = tile;                 // plain form
    u16* sK = tile + L * LDK;       // plain form
    float* sA = reinterpret_cast<float*>(sU);
    float* sT = sA + L * LDA;

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int c = blockIdx.x % p.nchunks;
    const int bh = blockIdx.x / p.nchunks;
    const int b = bh / p.H, h = bh - b * p.H;
    const int64_t T = p.T, t0 = static_cast<int64_t>(c) * L;
    const int K = p.K, H = p.H;

    const int64_t row_elems = static_cast<int64_t>(H) * K;
    const BufRes rq = make_rsrc(p.q + b * T * row_elems, T * row_elems * 2);
    const BufRes rk = make_rsrc(p.k + b * T * row_elems, T * row_elems * 2);
    // every load of the chunk is issued before the first LDS store, so the
    // memory latency is paid once, not once per piece
    constexpr int NPI = L * KP / 8 / NT;   // 16-byte q / k pieces per thread
    constexpr int NGE = DECAY ? L * KP / NT : 1;   // g elements per thread
    u32x4 xq[NPI], xk[NPI];
#pragma unroll
    for (int j = 0; j < NPI; ++j) {
        const int pi = tid + j * NT;
        const int row = pi / (KP / 8), c8 = (pi % (KP / 8)) * 8;
        const int64_t t = t0 + row;
        const int off = ((static_cast<int>(t) * H + h) * K + c8) * 2;
        const int64_t goff = ((b * T + t) * H + h) * static_cast<int64_t>(K);
        xq[j] = load_piece<VEC>(rq, p.q + goff, off, c8, K, t < T);
        xk[j] = load_piece<VEC>(rk, p.k + goff, off, c8, K, t < T);
    }
    // g rows of the chunk (zero past T and past K: no decay there); with
    // vector loads four keys per lane and load (a quarter of the instructions)
    float xg[NGE];
    if constexpr (DECAY) {
        if constexpr (VEC) {
            const BufRes rg = make_rsrc(p.g + b * T * row_elems, T * row_elems * 4);
#pragma unroll
            for (int j = 0; j < NGE / 4; ++j) {
                const int e = 4 * (tid + j * NT), row = e / KP, i = e % KP;
                const int off = (t0 + row < T && i < K) ? ((static_cast<int>(t0) + row) * H * K + h * K + i) * 4 : kBufOOB;
                const f32x4 x = __builtin_bit_cast(f32x4, buf_load16(rg, off));
#pragma unroll
                for (int r = 0; r < 4; ++r) xg[4 * j + r] = x[r];
            }
        } else {
#pragma unroll
            for (int j = 0; j < NGE; ++j) {
                const int e = tid + j * NT, row = e / KP, i = e % KP;
                const int64_t t = t0 + row;
                xg[j] = (t < T && i < K) ? p.g[((b * T + t) * H + h) * static_cast<int64_t>(K) + i] : 0.0f;
            }
        }
    }
    const float xb = (tid < L && t0 + tid < T) ? p.beta[(b * T + t0 + tid) * H + h] : 0.0f;
    if constexpr (!DECAY) {
#pragma unroll
        for (int j = 0; j < NPI; ++j) {
            const int pi = tid + j * NT;
            const int row = pi / (KP / 8), c8 = (pi % (KP / 8)) * 8;
            *reinterpret_cast<u32x4*>(sQ + row * LDK + c8) = xq[j];
            *reinterpret_cast<u32x4*>(sK + row * LDK + c8) = xk[j];
        }
    }
    if (tid < L) sBeta[tid] = xb;
    // decayed form: the raw q and k stay in the registers they were loaded into
    float* sG = reinterpret_cast<float*>(sU + G_OFF);
    if constexpr (DECAY) {
        if constexpr (VEC) {
#pragma unroll
            for (int j = 0; j < NGE / 4; ++j) {
                const int e = 4 * (tid + j * NT);
                *reinterpret_cast<f32x4*>(sG + (e / KP) * LDG + e % KP) =
                    f32x4{xg[4 * j], xg[4 * j + 1], xg[4 * j + 2], xg[4 * j + 3]};
            }
        } else {
#pragma unroll
            for (int j = 0; j < NGE; ++j) {
                const int e = tid + j * NT;
                sG[(e / KP) * LDG + e % KP] = xg[j];
            }
        }
    }
    __syncthreads();

    // A = K K^T and M = Q K^T lower-triangle blocks (20 jobs over 4 waves), kept in registers
    f32x4 acc[5];
    bf16x8 khh[DECAY ? NPI : 1], khl[DECAY ? NPI : 1];   // decayed form: khat pieces, hi/lo
    if constexpr (DECAY) {
        // running sum over the chunk per key: wave w sums rows 16w .. 16w+15 of
        // keys lane, lane + 64, ...
        constexpr int KPL = KP / 64;   // keys per lane
        float gl[KPL][16];
#pragma unroll
        for (int kk = 0; kk < KPL; ++kk) {
            const int key = lane + 64 * kk;
#pragma unroll
            for (int r = 0; r < 16; ++r) gl[kk][r] = sG[(16 * wave + r) * LDG + key];
#pragma unroll
            for (int r = 1; r < 16; ++r) gl[kk][r] += gl[kk][r - 1];
            sTot[wave][key] = gl[kk][15];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < KPL; ++kk) {
            const int key = lane + 64 * kk;
            float off = 0.0f;
            for (int w2 = 0; w2 < wave; ++w2) off += sTot[w2][key];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                gl[kk][r] += off;
                sG[(16 * wave + r) * LDG + key] = gl[kk][r];
            }
            if (wave == 1) sRef[key] = gl[kk][15];   // the middle step's running sum
        }
        __syncthreads();
        float dev = 0.0f;
#pragma unroll
        for (int kk = 0; kk < KPL; ++kk) {
            const float ref = sRef[lane + 64 * kk];
            if (wave == 0) dev = fmaxf(dev, fabsf(ref));   // G_{-1} = 0
#pragma unroll
            for (int r = 0; r < 16; ++r) dev = fmaxf(dev, fabsf(gl[kk][r] - ref));
        }
        const bool fast = !__syncthreads_or(dev > kHalfSpan);
        u16* tAh = tile;                 // a hi, later qt hi (half the keys)
        u16* tAl = tile + L * KH;        // a lo, later qt lo
        u16* tBh = tile + 2 * L * KH;
        u16* tBl = tile + 3 * L * KH;
        {
            // the scan's operands, relative to the chunk start: a = e^{G_{t-1}} k and
            // qt = e^{G_t} q as hi/lo planes, e^{G_L}, and khat = e^{G_L - G_t} k (kept
            // in registers for W); every exponent is <= 0 while g <= 0
            u16* blk = p.ws + static_cast<int64_t>(blockIdx.x) * chunk_u16<KP, true>();
            u16* aq = blk + off_aq<KP>();
#pragma unroll
            for (int j = 0; j < NPI; ++j) {
                const int pc = tid + j * NT, t = pc / (KP / 8), i0 = (pc % (KP / 8)) * 8;
                const u32x4 kw = xk[j];
                const u32x4 qw = xq[j];
                float av[8], qv[8], kv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float gt = sG[t * LDG + i0 + e], gp = t > 0 ? sG[(t - 1) * LDG + i0 + e] : 0.0f;
                    const float gL = sG[(L - 1) * LDG + i0 + e];
                    const float kx = bf2f(piece_elem(kw, e));
                    av[e] = kx * __expf(gp);
                    qv[e] = bf2f(piece_elem(qw, e)) * __expf(gt);
                    kv[e] = kx * __expf(gL - gt);
                }
                bf16x8 hi, lo;
                split8(av, hi, lo);
                *reinterpret_cast<bf16x8*>(aq + t * KP + i0) = hi;
                *reinterpret_cast<bf16x8*>(aq + L * KP + t * KP + i0) = lo;
                split8(qv, hi, lo);
                *reinterpret_cast<bf16x8*>(aq + 2 * L * KP + t * KP + i0) = hi;
                *reinterpret_cast<bf16x8*>(aq + 3 * L * KP + t * KP + i0) = lo;
                split8(kv, khh[j], khl[j]);
            }
            if (tid < KP) reinterpret_cast<float*>(blk + off_el<KP>())[tid] = __expf(sG[(L - 1) * LDG + tid]);
        }
        if (fast) {
            // per key range (all keys, or one half at K = 128): a = e^{G_{t-1} - ref} k
            // and b = e^{ref - G_t} k as hi/lo (eight keys of one step per piece, the
            // raw k in registers), A += a b^T; then qt = e^{G_t - ref} q into a's
            // tiles, M += qt b^T
            constexpr int NPC = L * KP / 8 / NT;
#pragma unroll
            for (int m = 0; m < 5; ++m) acc[m] = zero4();
            auto blocks = [&](bool want_m) {
#pragma unroll
                for (int m = 0; m < 5; ++m) {
                    const int n = wave + 4 * m;
                    if ((n >= 10) != want_m) continue;
                    int bi, bj;
                    tri_block(n % 10, bi, bj);
                    f32x4 a = acc[m];
#pragma unroll
                    for (int k0 = 0; k0 < KH; k0 += 32) {
                        const bf16x8 xh = tfrag<KH>(tAh, 16 * bi, k0, lane), xl = tfrag<KH>(tAl, 16 * bi, k0, lane);
                        const bf16x8 yh = tfrag<KH>(tBh, 16 * bj, k0, lane), yl = tfrag<KH>(tBl, 16 * bj, k0, lane);
                        a = mfma16(xl, yh, a);
                        a = mfma16(xh, yl, a);
                        a = mfma16(xh, yh, a);
                    }
                    acc[m] = a;
                }
            };
#pragma unroll
            for (int hh = 0; hh < NHALF; ++hh) {
#pragma unroll
                for (int j = 0; j < NPC; ++j) {
                    const int pc = tid + j * NT, t = pc / (KP / 8), i0 = (pc % (KP / 8)) * 8;
                    if (i0 / KH != hh) continue;
                    const u32x4 kw = xk[j];
                    float av[8], bv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float r0 = sRef[i0 + e];
                        const float gt = sG[t * LDG + i0 + e], gp = t > 0 ? sG[(t - 1) * LDG + i0 + e] : 0.0f;
                        const float kv = bf2f(piece_elem(kw, e));
                        av[e] = kv * __expf(gp - r0);
                        bv[e] = kv * __expf(r0 - gt);
                    }
                    bf16x8 hi, lo;
                    const int o = tswz<KH>(t, i0 - hh * KH);
                    split8(av, hi, lo);
                    *reinterpret_cast<bf16x8*>(tAh + o) = hi;
                    *reinterpret_cast<bf16x8*>(tAl + o) = lo;
                    split8(bv, hi, lo);
                    *reinterpret_cast<bf16x8*>(tBh + o) = hi;
                    *reinterpret_cast<bf16x8*>(tBl + o) = lo;
                }
                __syncthreads();
                blocks(false);
                __syncthreads();   // a is read: its tiles take qt
#pragma unroll
                for (int j = 0; j < NPC; ++j) {
                    const int pc = tid + j * NT, t = pc / (KP / 8), i0 = (pc % (KP / 8)) * 8;
                    if (i0 / KH != hh) continue;
                    const u32x4 qw = xq[j];
                    float qv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        qv[e] = bf2f(piece_elem(qw, e)) * __expf(sG[t * LDG + i0 + e] - sRef[i0 + e]);
                    bf16x8 hi, lo;
                    const int o = tswz<KH>(t, i0 - hh * KH);
                    split8(qv, hi, lo);
                    *reinterpret_cast<bf16x8*>(tAh + o) = hi;
                    *reinterpret_cast<bf16x8*>(tAl + o) = lo;
                }
                __syncthreads();
                blocks(true);
                if (hh + 1 < NHALF) __syncthreads();   // the tiles take the second half
            }
        } else {
            // strong decay: each needed entry from its pairs, exact exponentials
            // (the raw k and q as full-width tiles over the a and b half tiles)
            u16* const tK = tAh;   // [L][KP], spans tAh and tAl
            u16* const tQ = tBh;   // [L][KP], spans tBh and tBl
#pragma unroll
            for (int j = 0; j < NPI; ++j) {
                const int pc = tid + j * NT, t = pc / (KP / 8), i0 = (pc % (KP / 8)) * 8;
                *reinterpret_cast<u32x4*>(tK + tswz<KP>(t, i0)) = xk[j];
                *reinterpret_cast<u32x4*>(tQ + tswz<KP>(t, i0)) = xq[j];
            }
            __syncthreads();
#pragma unroll
            for (int m = 0; m < 5; ++m) {
                const int n = wave + 4 * m;
                int bi, bj;
                tri_block(n % 10, bi, bj);
                const int tau = 16 * bj + c16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * bi + 4 * g + r;
                    float sum = 0.0f;
                    if (n < 10 ? tau < t : tau <= t) {
                        const u16* ltile = n < 10 ? tK : tQ;
                        const float* gl_row = n < 10 ? sG + (t - 1) * LDG : sG + t * LDG;   // t >= 1 when n < 10
                        for (int i = 0; i < KP; ++i)
                            sum += bf2f(ltile[tswz<KP>(t, i)]) * bf2f(tK[tswz<KP>(tau, i)]) *
                                   __expf(gl_row[i] - sG[tau * LDG + i]);
                    }
                    acc[m][r] = sum;
                }
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < 5; ++m) {
            const int n = wave + 4 * m;
            int bi, bj;
            tri_block(n % 10, bi, bj);
            const u16* left = n < 10 ? sK : sQ;
            f32x4 a = zero4();
#pragma unroll
            for (int k0 = 0; k0 < KP; k0 += 32)
                a = mfma16(frag<LDK>(left, 16 * bi, k0, lane), frag<LDK>(sK, 16 * bj, k0, lane), a);
            acc[m] = a;
        }
    }
    __syncthreads();   // sQ / sK (decayed form: the tiles) are overwritten by sA / sT below
    // A into LDS now; the blocks of M stay in registers until T's space is free
#pragma unroll
    for (int m = 0; m < 5; ++m) {
        const int n = wave + 4 * m;
        if (n >= 10) continue;
        int bi, bj;
        tri_block(n, bi, bj);
        const int tau = 16 * bj + c16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * bi + 4 * g + r;
            sA[t * LDA + tau] = tau < t ? sBeta[t] * acc[m][r] : 0.0f;
        }
    }
    __syncthreads();

    // diagonal 16x16 blocks of T = (I + A)^{-1}: one lane per column
    if (wave == 0) {
        const int bk = lane / 16, col = lane % 16;
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

    // off-diagonal blocks of T: column block j = wave, block rows i = j+1..3,
    //   T_ij = -T_ii * sum_{m=j}^{i-1} A_im T_mj
    // A wave's LDS writes are visible to its own later LDS reads, so a column
    // block needs no barrier.
    if (wave < 3) {
        const int j = wave;
        for (int i = j + 1; i < 4; ++i) {
            f32x4 X = zero4();
            for (int m = j; m < i; ++m) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(sA + (16 * i + c16) * LDA + 16 * m + 4 * g);
                f32x4 bcol;
#pragma unroll
                for (int r = 0; r < 4; ++r) bcol[r] = sT[(16 * m + 4 * g + r) * LDA + 16 * j + c16];
                X = mm16(a, bcol, X);
            }
            const f32x4 tii = *reinterpret_cast<const f32x4*>(sT + (16 * i + c16) * LDA + 16 * i + 4 * g);
            const f32x4 Y = mm16(tii, X, zero4());
#pragma unroll
            for (int r = 0; r < 4; ++r) sT[(16 * i + 4 * g + r) * LDA + 16 * j + c16] = -Y[r];
        }
    }
    __syncthreads();

    // Tb = T diag(beta), transposed ([step'][step], zero above the diagonal of T)
    // and split hi/lo into A's space: the right operand of the MTb and W
    // products, read four steps at a time
    constexpr int LDT = L + 4;   // u16 row stride: 8-byte aligned rows
    static_assert(2 * L * LDT * 2 <= L * LDA * 4, "Tb^T tiles fit in A's space");
    u16* tTh = reinterpret_cast<u16*>(sA);
    u16* tTl = tTh + L * LDT;
    {
        // one 4x4 block per thread: rows tau = 4 a4 .., columns tp = 4 b4 .. of T,
        // transposed in registers and written four steps at a time
        static_assert(NT == (L / 4) * (L / 4), "one 4x4 block of T per thread");
        const int a4 = tid / (L / 4), b4 = tid % (L / 4);
        const f32x4 bt = *reinterpret_cast<const f32x4*>(sBeta + 4 * b4);
        f32x4 rows[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) rows[i] = *reinterpret_cast<const f32x4*>(sT + (4 * a4 + i) * LDA + 4 * b4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u16 hi[4], lo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = 4 * a4 + i >= 4 * b4 + j ? rows[i][j] * bt[j] : 0.0f;
                split_bf16(x, hi[i], lo[i]);
            }
            store4(tTh + (4 * b4 + j) * LDT + 4 * a4, hi[0], hi[1], hi[2], hi[3]);
            store4(tTl + (4 * b4 + j) * LDT + 4 * a4, lo[0], lo[1], lo[2], lo[3]);
        }
    }
    __syncthreads();

    // M into T's space, which the staging above has consumed (so the kernel
    // needs no separate M buffer: a smaller LDS footprint, more workgroups per CU)
    float* sM = sT;
#pragma unroll
    for (int m = 0; m < 5; ++m) {
        const int n = wave + 4 * m;
        if (n < 10) continue;
        int bi, bj;
        tri_block(n - 10, bi, bj);
        const int tau = 16 * bj + c16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * bi + 4 * g + r;
            sM[t * LDA + tau] = tau <= t ? acc[m][r] : 0.0f;
        }
    }
    __syncthreads();

    u16* blk = p.ws + static_cast<int64_t>(blockIdx.x) * chunk_u16<KP, DECAY>();
    // MTb lower blocks (i, j): (sum_{m=j}^{i} M_im T_mj) diag(beta); five block
    // products per wave, formed transposed (Tb^T M^T) so that each lane holds
    // four consecutive columns of one row: one 8-byte store per plane
    {
        for (int qj = 0; qj < 4; ++qj) {
            int bi, bj;
            mtb_job(wave, qj, bi, bj);
            if (bi < 0) continue;
            f32x4 X = zero4();
            for (int m = bj; m <= bi; ++m) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(sM + (16 * bi + c16) * LDA + 16 * m + 4 * g);
                const int to = (16 * bj + c16) * LDT + 16 * m + 4 * g;
                X = mm16_la(*reinterpret_cast<const s16x4*>(tTh + to), *reinterpret_cast<const s16x4*>(tTl + to), a, X);
            }
            // X[r]: row 16 bi + c16, column 16 bj + 4 g + r: fragment lane
            // c16 + 16 (2 (bj % 2) + g / 2), elements 4 (g % 2) + r of block (bi, bj / 2)
            u16 hi[4], lo[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) split_bf16(X[r], hi[r], lo[r]);
            const int idx = mfrag_off(bi, bj >> 1, 0) + (c16 + 16 * (2 * (bj & 1) + (g >> 1))) * 8 + 4 * (g & 1);
            store4(blk + idx, hi[0], hi[1], hi[2], hi[3]);
            store4(blk + idx + 512, lo[0], lo[1], lo[2], lo[3]);
        }
        // zeros for the blocks right of the diagonal that the scan reads: (0, 1)
        // and (2, 3), the upper halves (lanes 32 ..) of blocks (0, 0) and (2, 1)
        if (tid < 128) {
            const int rb = (tid >> 6) * 2, hl = (tid >> 5) & 1, lp = 32 + (tid & 31);
            const u32x4 z = {0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(blk + mfrag_off(rb, rb >> 1, hl) + lp * 8) = z;
        }
    }
    __syncthreads();   // M is read: its space takes khat
    // W = khat^T Tb (key-major, [KP][L]); khat = k (plain form, exact in
    // bf16) or e^{G_L - G_t} k (decayed form, hi/lo), staged [step][key] in M's
    // space, or past sA and sT where it does not fit there (decayed, K = 128)
    {
        static_assert(!KH_PAST || U_BYTES - AT_BYTES >= KHAT_BYTES, "khat fits past sA and sT");
        u16* sKh = KH_PAST ? reinterpret_cast<u16*>(sU + AT_BYTES) : reinterpret_cast<u16*>(sM);
        u16* sKl = sKh + L * KP;
#pragma unroll
        for (int j = 0; j < NPI; ++j) {
            const int pc = tid + j * NT, t = pc / (KP / 8), i0 = (pc % (KP / 8)) * 8;
            if constexpr (DECAY) {
                *reinterpret_cast<bf16x8*>(sKh + t * KP + i0) = khh[j];
                *reinterpret_cast<bf16x8*>(sKl + t * KP + i0) = khl[j];
            } else {
                *reinterpret_cast<u32x4*>(sKh + t * KP + i0) = xk[j];
            }
        }
        __syncthreads();
        u16* wh = blk + off_w<KP>();
        for (int n = wave; n < KP / 16 * 4; n += 4) {
            const int ib = n / 4, jb = n % 4;   // key block, step block
            f32x4 acc2 = zero4();
            for (int m = jb; m < 4; ++m) {
                // right: khat (column = key 16 ib + c16, k = step 16 m + 4 g + e);
                // left: Tb^T (row = step 16 jb + c16, same k), lower blocks only;
                // the transposing LDS read: lane i of a 16-lane group supplies step
                // 16 m + 4 g + i / 4, keys 16 ib + 4 (i % 4) .. +3; lane j receives
                // khat[16 m + 4 g .. +3][16 ib + j]
                const int xoff = (16 * m + 4 * g + (c16 >> 2)) * KP + 16 * ib + 4 * (c16 & 3);
                const s16x4 xh = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sKh + xoff));
                s16x4 xl;
                if constexpr (DECAY) xl = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sKl + xoff));
                const int to = (16 * jb + c16) * LDT + 16 * m + 4 * g;
                const s16x4 yh = *reinterpret_cast<const s16x4*>(tTh + to);
                const s16x4 yl = *reinterpret_cast<const s16x4*>(tTl + to);
                // formed transposed (Tb^T khat): the left operand is Tb^T, the right khat
                if constexpr (DECAY) acc2 = mfma16k16(yh, xl, acc2);
                acc2 = mfma16k16(yl, xh, acc2);
                acc2 = mfma16k16(yh, xh, acc2);
            }
            // acc2[r]: key 16 ib + c16, step 16 jb + 4 g + r
            u16 hi[4], lo[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) split_bf16(acc2[r], hi[r], lo[r]);
            // steps 16 jb + 4 g + r: fragment lane c16 + 16 (2 (jb % 2) + g / 2),
            // elements 4 (g % 2) + r of block (ib, jb / 2)
            const int idx = wfrag_off(ib, jb >> 1, 0) + (c16 + 16 * (2 * (jb & 1) + (g >> 1))) * 8 + 4 * (g & 1);
            store4(wh + idx, hi[0], hi[1], hi[2], hi[3]);
            store4(wh + idx + 512, lo[0], lo[1], lo[2], lo[3]);
        }
    }
}

// ---------------------------------------------------------------------------
// scan: sequential over chunks per (batch, head, 16-wide V-tile)
// ---------------------------------------------------------------------------
// Byte offset of 16-byte piece `p` of row `r` in a row-major tile whose rows
// hold PPR pieces, with the pieces of each row rotated by an XOR of the row
// index: 16 consecutive rows read at one column then hit different banks.
template <int PPR>
__device__ __forceinline__ int swz(int r, int p) {
    return r * (PPR * 16) + ((p ^ (r & (PPR - 1))) << 4);
}

// Wave w owns chunk rows 16w .. 16w+15 (Y, R, outputs) and state keys
// 16 STW w .. (row tiles of S).  The chunk's operand tiles (q and k; decayed
// form: a and qt as hi/lo) and the V tile sit in LDS as swizzled tiles read
// as matrix-core operands (one stage each with vector loads, two by chunk
// parity on the scalar path).  W, MTb (and
// e^{G_L}) go straight to registers as operand fragments: each wave reads
// only the W rows of its own state keys and the MTb rows of its own chunk
// rows, as contiguous 1 KB fragments.  With vector loads all of the next
// chunk's loads are issued at the top of a chunk: the operand and V tiles
// into registers, written to LDS at the chunk's end (after the middle
// barrier, no wave reads the chunk's own tiles any more); W and MTb
// into the other of two register sets (the chunk loop is unrolled twice, so
// the sets alternate with no copies).  The first chunk's tiles come through
// loads with an LDS destination.  Per chunk, two barriers:
//   -- inputs of chunk c visible --
//   1. Y = K S0, O1 = Q S0 (rows of this wave); R = V - Y -> LDS
//   -- barrier --
//   2. O = scale (O1 + MTb R) -> outputs; S = D S0 + W R (tiles of this wave)
//      -> LDS as the next chunk's operand
// The decayed form at K = 128 has 64 KB of operand tiles per chunk, too much
// to stage through registers beside the rest: each wave loads the next
// chunk's rows of its own (the only rows it reads) with
// LDS-destination loads as soon as its step 1 is done with them, so they
// load during step 2.
// SEGP = false: outputs of segment s from the state entering it (all
// segments at once; the last writes s_final).  SEGP = true, the segment pass:
// no readout; segment 0 runs its state columns from s0 and leaves the state
// entering segment 1, and a segment s in 1 .. nseg - 2 runs K identity
// columns with zero values (A_s) beside its state columns from zero (B_s).
template <int KP, bool VEC, bool DECAY, bool SEGP = false>
__global__ __launch_bounds__(NT) void delta_scan_kernel(DeltaArgs p) {
    static_assert(!DECAY || KP == 64 || KP == KD, "decayed form: K <= 128");
    constexpr bool SPLIT = DECAY && KP > 64;   // operand tiles single buffered
    constexpr int PPR = KP / 8;          // 16-byte pieces per operand row
    constexpr int QB = L * KP * 2;       // bytes of one [L][KP] bf16 operand tile
    constexpr int PB = L * L * 2;        // bytes of an MTb plane
    constexpr int VB = L * VT * 2;       // bytes of the V tile
    constexpr int NOPS = DECAY ? 4 : 2;  // operand tiles: q, k; or a hi, a lo, qt hi, qt lo
    constexpr int OFF_AH = DECAY ? 0 : QB, OFF_AL = QB;        // k (a hi, a lo)
    constexpr int OFF_QH = DECAY ? 2 * QB : 0, OFF_QL = 3 * QB;   // q (qt hi, qt lo)
    constexpr int OPS = NOPS * QB;       // operand stage
    constexpr int OFF_V = 0;
    constexpr int PVS = OFF_V + VB;      // V stage
    // load runs per wave and chunk (vector loads): operand tiles, MTb planes
    constexpr int NJ_OPS = SPLIT ? 4 * 16 * PPR / 64 : (DECAY ? 4 : 1) * QB / 4096;
    constexpr int CHUNK_BYTES = chunk_u16<KP, DECAY>() * 2;
    constexpr int LDK = KP + 8;
    constexpr int LDL = L + 8;
    constexpr int KS = KP / 32;          // k-steps over the key dimension
    constexpr int STW = KP / 16 / 4;     // state row tiles per wave
    static_assert(STW >= 1, "state tiles");
    static_assert(QB % 1024 == 0 && PB % 1024 == 0 && VB == 2048, "1 KB load runs");

    // Stages: with vector loads the next chunk's tiles are written at the end of
    // a chunk, after its middle barrier, when no wave reads the chunk's own
    // tiles any more: one stage of each.  The scalar path loads the next
    // chunk's tiles into LDS during the chunk: two stages, by chunk parity.
    constexpr int NSO = (SPLIT || VEC) ? 1 : 2, NSV = VEC ? 1 : 2;
    __shared__ __align__(16) unsigned char sOps[NSO * OPS];
    __shared__ __align__(16) unsigned char sPV[NSV * PVS];
    __shared__ __align__(16) u16 sRTh[VT * LDL];     // R^T hi/lo
    __shared__ __align__(16) u16 sRTl[VT * LDL];
    __shared__ __align__(16) u16 sSh[VT * LDK];      // S^T hi/lo entering the chunk
    __shared__ __align__(16) u16 sSl[VT * LDK];
    constexpr int LDO = 20;                          // fp32 row stride of the output tiles
    __shared__ __align__(16) float sO[4][16 * LDO];  // each wave's 16 x 16 output tile

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
    // (batch, head, segment, tile): output pass V-tiles of every segment; the
    // segment pass V-tiles of segment 0, then for each segment 1 .. nseg - 2
    // its ceil(K / 16) A tiles and its V-tiles
    int bh, seg, vt;
    bool atile = false;   // segment pass: this tile runs identity columns (A_s)
    if constexpr (SEGP) {
        const int kt = (p.K + VT - 1) / VT;
        const int per = p.vtiles + (p.nseg - 2) * (kt + p.vtiles);
        bh = lid / per;
        const int r = lid - bh * per;
        if (r < p.vtiles) {
            seg = 0;
            vt = r;
        } else {
            seg = 1 + (r - p.vtiles) / (kt + p.vtiles);
            const int t = (r - p.vtiles) % (kt + p.vtiles);
            atile = t < kt;
            vt = atile ? t : t - kt;
        }
    } else {
        vt = lid % p.vtiles;
        const int rest = lid / p.vtiles;
        seg = rest % p.nseg;
        bh = rest / p.nseg;
    }
    const int b = bh / p.H, h = bh - b * p.H;
    const int64_t T = p.T;
    const int K = p.K, V = p.V, H = p.H;
    // identity columns read no values: their V-tile starts past V
    const int v0 = atile ? V : vt * VT;
    const int nchunks = p.nchunks;
    const int c_begin = seg * p.cps;
    const int c_end = min(c_begin + p.cps, nchunks);

    const int64_t qk_row = static_cast<int64_t>(H) * K * 2, v_row = static_cast<int64_t>(H) * V * 2;   // bytes per step
    const u16* qb = p.q + b * T * H * static_cast<int64_t>(K);
    const u16* kb = p.k + b * T * H * static_cast<int64_t>(K);
    const u16* vb = p.v + b * T * H * static_cast<int64_t>(V);
    const u16* wsb = p.ws + static_cast<int64_t>(bh) * nchunks * chunk_u16<KP, DECAY>();
    const int64_t ws_bytes = static_cast<int64_t>(nchunks) * CHUNK_BYTES;

    // ---- fetch of one chunk's LDS operands ----
    // Load run i (64 lanes x 16 bytes) fills bytes 1024 i .. of a tile: lane l
    // takes slot s = 64 i + l, i.e. row s / PPR, stored piece s % PPR, which
    // holds the row's piece (s % PPR) ^ (row & (PPR - 1)).
    // Operand tiles into `so_`; all rows, or (SPLIT) this wave's 16.  With
    // vector loads a wave issues its NJ_OPS runs (a run: one load instruction
    // per operand tile of the plain form, one in all of the decayed form).
    auto fetch_ops = [&](int c, unsigned char* so_) {
        const int64_t t0 = static_cast<int64_t>(c) * L;
        if constexpr (VEC) {
            if constexpr (DECAY) {
                // a hi, a lo, qt hi, qt lo: four [L][KP] tiles, back to back in the workspace
                const BufRes wp = make_rsrc_window(wsb, ws_bytes, static_cast<int64_t>(c) * CHUNK_BYTES);
                if constexpr (SPLIT) {
                    constexpr int RPR = 64 / PPR;   // rows per run
#pragma unroll
                    for (int j = 0; j < NJ_OPS; ++j) {
                        const int tl = j / (16 / RPR), row0 = 16 * wave + RPR * (j % (16 / RPR));
                        const int row = row0 + lane / PPR, pc = (lane % PPR) ^ (row & (PPR - 1));
                        const int off = off_aq<KP>() * 2 + tl * QB + row * KP * 2 + pc * 16;
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            wp, (__attribute__((address_space(3))) void*)(so_ + tl * QB + row0 * KP * 2), 16, off,
                            0, 0, 0);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < NJ_OPS; ++j) {
                        const int i = wave + 4 * j, tl = i / (QB / 1024), sl = 64 * (i % (QB / 1024)) + lane;
                        const int row = sl / PPR, pc = (sl % PPR) ^ (row & (PPR - 1));
                        const int off = off_aq<KP>() * 2 + tl * QB + row * KP * 2 + pc * 16;
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            wp, (__attribute__((address_space(3))) void*)(so_ + 1024 * i), 16, off, 0, 0, 0);
                    }
                }
            } else {
                const BufRes wq = make_rsrc_window(qb, T * qk_row, t0 * qk_row);
                const BufRes wk = make_rsrc_window(kb, T * qk_row, t0 * qk_row);
#pragma unroll
                for (int j = 0; j < NJ_OPS; ++j) {
                    const int i = wave + 4 * j, sl = 64 * i + lane;
                    const int row = sl / PPR, col = ((sl % PPR) ^ (row & (PPR - 1))) * 8;
                    const int off = col < K ? ((row * H + h) * K + col) * 2 : kBufOOB;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        wq, (__attribute__((address_space(3))) void*)(so_ + OFF_QH + 1024 * i), 16, off, 0, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        wk, (__attribute__((address_space(3))) void*)(so_ + OFF_AH + 1024 * i), 16, off, 0, 0, 0);
                }
            }
        } else {
            // same slots, filled through registers (odd sizes or alignment)
            if constexpr (DECAY) {
                const unsigned char* aw = reinterpret_cast<const unsigned char*>(
                    wsb + static_cast<int64_t>(c) * chunk_u16<KP, DECAY>() + off_aq<KP>());
                const int first = SPLIT ? lane : tid, step = SPLIT ? 64 : NT;
                for (int s2 = first; s2 < (SPLIT ? 4 * 16 * PPR : 4 * L * PPR); s2 += step) {
                    const int per = SPLIT ? 16 * PPR : L * PPR;
                    const int tl = s2 / per, sl = (SPLIT ? 16 * PPR * wave : 0) + s2 % per;
                    const int row = sl / PPR, pc = (sl % PPR) ^ (row & (PPR - 1));
                    *reinterpret_cast<u32x4*>(so_ + tl * QB + 16 * sl) =
                        *reinterpret_cast<const u32x4*>(aw + tl * QB + row * KP * 2 + pc * 16);
                }
            } else {
                for (int sl = tid; sl < L * PPR; sl += NT) {
                    const int row = sl / PPR, col = ((sl % PPR) ^ (row & (PPR - 1))) * 8;
                    const int64_t t = t0 + row;
                    u32x4 xq = {0u, 0u, 0u, 0u}, xk = {0u, 0u, 0u, 0u};
                    if (t < T) {
                        const int64_t o = (t * H + h) * static_cast<int64_t>(K);
                        xq = load8_bf16(qb + o, col, K, false);
                        xk = load8_bf16(kb + o, col, K, false);
                    }
                    *reinterpret_cast<u32x4*>(so_ + OFF_QH + 16 * sl) = xq;
                    *reinterpret_cast<u32x4*>(so_ + OFF_AH + 16 * sl) = xk;
                }
            }
        }
    };
    // the V tile into `sp_`
    auto fetch_pv = [&](int c, unsigned char* sp_) {
        const int64_t t0 = static_cast<int64_t>(c) * L;
        if constexpr (VEC) {
            const BufRes wv = make_rsrc_window(vb, T * v_row, t0 * v_row);
            if (wave < 2) {
                const int sl = 64 * wave + lane, row = sl / 2, col = ((sl % 2) ^ (row & 1)) * 8;
                const int off = v0 + col < V ? ((row * H + h) * V + v0 + col) * 2 : kBufOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    wv, (__attribute__((address_space(3))) void*)(sp_ + OFF_V + 1024 * wave), 16, off, 0, 0, 0);
            }
        } else {
            if (tid < L * 2) {
                const int row = tid / 2, col = ((tid % 2) ^ (row & 1)) * 8;
                const int64_t t = t0 + row;
                u32x4 xv = {0u, 0u, 0u, 0u};
                if (t < T) xv = load8_bf16(vb + (t * H + h) * static_cast<int64_t>(V) + v0, col, V - v0, false);
                *reinterpret_cast<u32x4*>(sp_ + OFF_V + 16 * tid) = xv;
            }
        }
    };

    // ---- register-staged prefetch of the next chunk (vector loads) ----
    // The same 16-byte slots as the LDS-direct loads above, loaded into
    // registers during a chunk and written to LDS at its end.
    // (An LDS-direct load in flight makes the compiler wait for it before any
    // later LDS read it cannot tell apart, which would expose the prefetch.)
    // Plain form: q and k pieces of runs 0 .. QB/4096 - 1; decayed form (not
    // SPLIT): the four operand tiles' runs; then the V tile.
    constexpr int NPO = SPLIT ? 1 : (DECAY ? 4 : 2) * QB / 4096;
    constexpr int NJO = DECAY ? NPO : NPO / 2;   // runs of preload_ops
    // DRAIN: the V piece is issued last, so its wait at the end of a chunk
    // waits for all of the next chunk's loads.  At K = 128 (~84 KB per chunk)
    // the loads take longer than the chunk's chain, and loads still in flight
    // into the next chunk delay that chunk's own (measured slower), and the
    // decayed form at K = 64 measured no better without it; in the plain form
    // at K = 64 the W / MTb loads may stay in flight until the next chunk's
    // phase 2.
    constexpr bool DRAIN = KP > 64 || DECAY;
    u32x4 pre_o[NPO], pre_v;
    auto preload_ops = [&](int c, int j0, int j1) {
        if constexpr (DECAY) {
            const BufRes wp = make_rsrc_window(wsb, ws_bytes, static_cast<int64_t>(c) * CHUNK_BYTES);
#pragma unroll
            for (int j = j0; j < j1; ++j) {
                const int i = wave + 4 * j, tl = i / (QB / 1024), sl = 64 * (i % (QB / 1024)) + lane;
                const int row = sl / PPR, pc = (sl % PPR) ^ (row & (PPR - 1));
                pre_o[j] = buf_load16(wp, off_aq<KP>() * 2 + tl * QB + row * KP * 2 + pc * 16);
            }
        } else {
            const int64_t t0 = static_cast<int64_t>(c) * L;
            const BufRes wq = make_rsrc_window(qb, T * qk_row, t0 * qk_row);
            const BufRes wk = make_rsrc_window(kb, T * qk_row, t0 * qk_row);
#pragma unroll
            for (int j = j0; j < j1; ++j) {
                const int i = wave + 4 * j, sl = 64 * i + lane;
                const int row = sl / PPR, col = ((sl % PPR) ^ (row & (PPR - 1))) * 8;
                const int off = col < K ? ((row * H + h) * K + col) * 2 : kBufOOB;
                if constexpr (!SEGP) pre_o[2 * j] = buf_load16(wq, off);
                pre_o[2 * j + 1] = buf_load16(wk, off);
            }
        }
    };
    auto preload_v = [&](int c) {
        // issued by every wave (waves 2 and 3 read nothing), like every other load here
        const int64_t t0 = static_cast<int64_t>(c) * L;
        const BufRes wv = make_rsrc_window(vb, T * v_row, t0 * v_row);
        const int sl = 64 * wave + lane, row = sl / 2, col = ((sl % 2) ^ (row & 1)) * 8;
        pre_v = buf_load16(wv, wave < 2 && v0 + col < V ? ((row * H + h) * V + v0 + col) * 2 : kBufOOB);
    };
    auto prestore = [&](unsigned char* so_, unsigned char* sp_) {
        if constexpr (!SPLIT) {
#pragma unroll
            for (int j = 0; j < (DECAY ? NPO : NPO / 2); ++j) {
                const int i = wave + 4 * j;
                if constexpr (DECAY) {
                    *reinterpret_cast<u32x4*>(so_ + 1024 * i + 16 * lane) = pre_o[j];
                } else {
                    if constexpr (!SEGP) *reinterpret_cast<u32x4*>(so_ + OFF_QH + 1024 * i + 16 * lane) = pre_o[2 * j];
                    *reinterpret_cast<u32x4*>(so_ + OFF_AH + 1024 * i + 16 * lane) = pre_o[2 * j + 1];
                }
            }
        }
        if (wave < 2) *reinterpret_cast<u32x4*>(sp_ + OFF_V + 1024 * wave + 16 * lane) = pre_v;
    };

    // ---- L2 touch of the (batch, head)'s shared lines, two chunks ahead ----
    // The vtiles workgroups of one (batch, head) read the same workspace
    // block and q / k rows, and each reads a slice of the same V rows: with
    // no one ahead, all of them wait on the same misses.  Each touches one
    // dword per 128-byte line of its 1/vtiles share of those lines two chunks
    // ahead, so that the register loads one chunk later hit in L2.  The
    // touched dwords are folded into a sink one chunk later (by then they
    // have arrived, so the fold does not wait) and kept live at the end.
    constexpr int LINE = 128;
    constexpr int NTOUCH = 2;   // touches per thread and chunk (a share of up to 512 lines)
    unsigned l2x[NTOUCH] = {0u, 0u}, l2sink = 0u;
    auto l2_touch = [&](int c) {
#pragma unroll
        for (int i = 0; i < NTOUCH; ++i) l2sink |= l2x[i];
        const int64_t t0 = static_cast<int64_t>(c) * L;
        const int lq = (K * 2 + LINE - 1) / LINE, lv = (V * 2 + LINE - 1) / LINE;   // lines per row
        const int n_ws = CHUNK_BYTES / LINE, n_qk = DECAY ? 0 : 2 * L * lq;
        const int n = n_ws + n_qk + L * lv;
        const int beg = vt * n / p.vtiles, end = (vt + 1) * n / p.vtiles;
        const BufRes wp = make_rsrc_window(wsb, ws_bytes, static_cast<int64_t>(c) * CHUNK_BYTES);
        const BufRes wq = make_rsrc_window(qb, T * qk_row, t0 * qk_row);
        const BufRes wk = make_rsrc_window(kb, T * qk_row, t0 * qk_row);
        const BufRes wv = make_rsrc_window(vb, T * v_row, t0 * v_row);
#pragma unroll
        for (int i = 0; i < NTOUCH; ++i) {
            const int x = beg + tid + NT * i;
            unsigned val = 0u;
            if (x < end) {
                if (x < n_ws) {
                    val = __builtin_amdgcn_raw_buffer_load_b32(wp, x * LINE, 0, 0);
                } else if (x < n_ws + n_qk) {
                    const int j = x - n_ws, r = (j % (L * lq)) / lq, li = j % lq;
                    const int off = r * static_cast<int>(qk_row) + h * K * 2 + min(li * LINE, K * 2 - 4);
                    val = __builtin_amdgcn_raw_buffer_load_b32(j < L * lq ? wq : wk, off, 0, 0);
                } else {
                    const int j = x - n_ws - n_qk, r = j / lv, li = j % lv;
                    const int off = r * static_cast<int>(v_row) + h * V * 2 + min(li * LINE, V * 2 - 4);
                    val = __builtin_amdgcn_raw_buffer_load_b32(wv, off, 0, 0);
                }
            }
            l2x[i] = val;
        }
    };

    // ---- W rows of this wave's state keys (and e^{G_L}), and the MTb rows
    // of its chunk rows, into registers ----
    // W frag (st, ks): key 16 sr + c16, steps 32 ks + 8 g .. +7; hi then lo.
    // MTb frag (ks): row 16 wave + c16, steps 32 ks + 8 g .. +7 (ks <= wave / 2)
    u32x4 wcur[STW][2][2], wnxt[STW][2][2], mcur[2][2], mnxt[2][2];
    f32x4 ecur[DECAY ? STW : 1], enxt[DECAY ? STW : 1];
    auto load_w = [&](int c, u32x4 (&w)[STW][2][2], f32x4 (&e)[DECAY ? STW : 1], u32x4 (&m)[2][2]) {
        const int64_t cb = static_cast<int64_t>(c) * CHUNK_BYTES;
        {
            // the workspace is the library's own (16-byte aligned): vector loads on both paths
            const BufRes wp = make_rsrc_window(wsb, ws_bytes, cb);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int hl = 0; hl < 2; ++hl)
                    m[ks][hl] = SEGP ? u32x4{0u, 0u, 0u, 0u}
                                     : buf_load16(wp, ks <= wave / 2 ? (mfrag_off(wave, ks, hl) + 8 * lane) * 2 : kBufOOB);
        }
        if constexpr (VEC) {
            const BufRes wp = make_rsrc_window(wsb, ws_bytes, cb);
#pragma unroll
            for (int st2 = 0; st2 < STW; ++st2) {
                const int kt = STW * wave + st2;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int hl = 0; hl < 2; ++hl)
                        w[st2][ks][hl] = buf_load16(wp, (off_w<KP>() + wfrag_off(kt, ks, hl) + 8 * lane) * 2);
                if constexpr (DECAY)
                    e[st2] = __builtin_bit_cast(f32x4, buf_load16(wp, off_el<KP>() * 2 + (16 * (STW * wave + st2) + 4 * g) * 4));
            }
        } else {
            const unsigned char* pw = reinterpret_cast<const unsigned char*>(wsb) + cb;
#pragma unroll
            for (int st2 = 0; st2 < STW; ++st2) {
                const int kt = STW * wave + st2;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int hl = 0; hl < 2; ++hl)
                        w[st2][ks][hl] = *reinterpret_cast<const u32x4*>(
                            pw + (off_w<KP>() + wfrag_off(kt, ks, hl) + 8 * lane) * 2);
                if constexpr (DECAY)
                    e[st2] = *reinterpret_cast<const f32x4*>(pw + off_el<KP>() * 2 + (16 * (STW * wave + st2) + 4 * g) * 4);
            }
        }
    };

    // state: wave owns row tiles sr = STW * wave + st (keys 16 sr .. 16 sr + 15)
    f32x4 S[STW];
    // the state entering the segment: s0 (segment 0), the one the prefix left
    // (output pass, segment >= 1), zero (segment pass B_s), identity (A_s)
    const float* sin = seg == 0 ? p.s0
                     : (SEGP ? nullptr : p.seg_state + (static_cast<int64_t>(seg) * p.B * H + bh) * K * V);
#pragma unroll
    for (int st = 0; st < STW; ++st) {
        const int sr = STW * wave + st;
        const int j = v0 + c16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = 16 * sr + 4 * g + r;
            float x = 0.0f;
            if (atile) x = d == 16 * vt + c16 ? 1.0f : 0.0f;
            else if (sin && d < K && j < V) x = sin[(seg == 0 ? (static_cast<int64_t>(b) * H + h) * K : 0) * V + d * V + j];
            S[st][r] = x;
        }
    }
    auto write_state_lds = [&]() {
#pragma unroll
        for (int st = 0; st < STW; ++st) {
            const int d = 16 * (STW * wave + st) + 4 * g;
            uint32_t hi[2], lo[2];
            split2(S[st][0], S[st][1], hi[0], lo[0]);
            split2(S[st][2], S[st][3], hi[1], lo[1]);
            *reinterpret_cast<u32x2*>(sSh + c16 * LDK + d) = u32x2{hi[0], hi[1]};
            *reinterpret_cast<u32x2*>(sSl + c16 * LDK + d) = u32x2{lo[0], lo[1]};
        }
    };
    write_state_lds();
    fetch_ops(c_begin, sOps + (NSO == 2 ? (c_begin & 1) * OPS : 0));
    fetch_pv(c_begin, sPV + (NSV == 2 ? (c_begin & 1) * PVS : 0));
    load_w(c_begin, wcur, ecur, mcur);
    if constexpr (VEC && DECAY)
        if (c_begin + 1 < c_end) l2_touch(c_begin + 1);

    const int arow = 16 * wave + c16;    // operand row of this wave
    // A chunk's outputs wait in this wave's LDS tile (rows 16 wave .., the 16
    // columns) and are stored during the next chunk, 16 bytes per lane (one
    // store instruction per wave instead of four of 4-byte pieces), so the wait
    // for this wave's loads at the top of a chunk does not wait on them.
    float* so = sO[wave];
    auto store_outputs = [&](int64_t tc) {
        const int row = lane >> 2, cc = 4 * (lane & 3), col = v0 + cc;
        const f32x4 x = *reinterpret_cast<const f32x4*>(so + row * LDO + cc);
        const int64_t t = tc + 16 * wave + row;
        if (t < T) {
            const int64_t oi = ((b * T + t) * H + h) * static_cast<int64_t>(V) + col;
            if (p.out_bf16) {
                u16* dst = reinterpret_cast<u16*>(p.o) + oi;
                if (VEC && col + 4 <= V) {
                    const uint32_t w0 = f2bf(x[0]) | (static_cast<uint32_t>(f2bf(x[1])) << 16);
                    const uint32_t w1 = f2bf(x[2]) | (static_cast<uint32_t>(f2bf(x[3])) << 16);
                    *reinterpret_cast<u32x2*>(dst) = u32x2{w0, w1};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < V) dst[e] = f2bf(x[e]);
                }
            } else {
                if (VEC && col + 4 <= V) {
                    *reinterpret_cast<f32x4*>(p.o + oi) = x;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < V) p.o[oi + e] = x[e];
                }
            }
        }
    };
    // One chunk; the W / MTb / e^{G_L} registers alternate between two sets
    // (this chunk's, the next chunk's) by unrolling the chunk loop twice, so no
    // copy at the end of a chunk waits for the next chunk's loads.
    auto step = [&](int c, u32x4 (&wc)[STW][2][2], f32x4 (&ec)[DECAY ? STW : 1], u32x4 (&mc)[2][2],
                    u32x4 (&wn)[STW][2][2], f32x4 (&en)[DECAY ? STW : 1], u32x4 (&mn)[2][2]) {
        const int64_t t0 = static_cast<int64_t>(c) * L;
        const unsigned char* st = sOps + (NSO == 2 ? (c & 1) * OPS : 0);
        const unsigned char* sp = sPV + (NSV == 2 ? (c & 1) * PVS : 0);
        const bool more = c + 1 < c_end;
        unsigned char* so_n = sOps + (NSO == 2 ? ((c + 1) & 1) * OPS : 0);
        unsigned char* sp_n = sPV + (NSV == 2 ? ((c + 1) & 1) * PVS : 0);
        // LDS-direct loads in flight (the first chunk's; SPLIT: every chunk's
        // operand rows) are waited for here; register-staged loads by their use
        if constexpr (VEC)
            if (SPLIT || c == c_begin) __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if constexpr (VEC) {
            // All of the next chunk's loads, issued here (past the last chunk
            // their windows are empty and read zero, so every chunk has the same
            // loads in flight and the compiler's waits are exact).
            if constexpr (!SPLIT) preload_ops(c + 1, 0, NJO);
            if constexpr (!DRAIN) preload_v(c + 1);
            load_w(c + 1, wn, en, mn);
            if constexpr (DRAIN) preload_v(c + 1);
        } else if (more) {
            load_w(c + 1, wn, en, mn);
            if constexpr (!SPLIT) fetch_ops(c + 1, so_n);
            fetch_pv(c + 1, sp_n);
        }
        if (!SEGP && c > c_begin) store_outputs(t0 - L);

        // ---- 1: Y = K S0, O1 = Q S0 (row block = wave), R = V - Y ----
        f32x4 y = zero4(), o1 = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 sh = frag<LDK>(sSh, 0, 32 * ks, lane);
            const bf16x8 sl = frag<LDK>(sSl, 0, 32 * ks, lane);
            const int po = swz<PPR>(arow, 4 * ks + g);
            const bf16x8 ah = *reinterpret_cast<const bf16x8*>(st + OFF_AH + po);
            if constexpr (DECAY) {
                const bf16x8 al = *reinterpret_cast<const bf16x8*>(st + OFF_AL + po);
                y = mfma16(al, sh, y);
                if constexpr (!SEGP) {
                    const bf16x8 ql = *reinterpret_cast<const bf16x8*>(st + OFF_QL + po);
                    o1 = mfma16(ql, sh, o1);
                }
            }
            y = mfma16(ah, sl, y);
            y = mfma16(ah, sh, y);
            if constexpr (!SEGP) {   // the segment pass has no readout
                const bf16x8 qh = *reinterpret_cast<const bf16x8*>(st + OFF_QH + po);
                o1 = mfma16(qh, sl, o1);
                o1 = mfma16(qh, sh, o1);
            }
        }
        {
            // V rows 16 wave + 4g .. +3 at column c16, by the transposing read
            const int vr = 16 * wave + 4 * g + (c16 >> 2), vc = 4 * (c16 & 3);
            const s16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(sp + OFF_V + swz<2>(vr, vc >> 3) + (vc & 4) * 2));
            float rr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) rr[r] = bf2f(static_cast<u16>(v4[r])) - y[r];
            uint32_t hi[2], lo[2];
            split2(rr[0], rr[1], hi[0], lo[0]);
            split2(rr[2], rr[3], hi[1], lo[1]);
            const int t = 16 * wave + 4 * g;
            *reinterpret_cast<u32x2*>(sRTh + c16 * LDL + t) = u32x2{hi[0], hi[1]};
            *reinterpret_cast<u32x2*>(sRTl + c16 * LDL + t) = u32x2{lo[0], lo[1]};
        }
        if constexpr (VEC) {
            if constexpr (DECAY)   // (the plain form's shared lines already hit in L2)
                if (c + 2 < c_end) l2_touch(c + 2);
        }
        __syncthreads();
        if constexpr (SPLIT) {
            // this wave's operand rows are read (y and o1 hold them; the
            // barrier waited for its LDS reads): the next chunk's may overwrite
            // them.  Issued after the barrier, which would otherwise wait for
            // these LDS-destination loads; the wait at the top of the next
            // chunk takes them instead, after step 2.
            if (more) fetch_ops(c + 1, sOps);
        }

        // ---- 2: O = scale (O1 + MTb R); S = D S0 + W R ----
        bf16x8 rh[2], rl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            rh[ks] = frag<LDL>(sRTh, 0, 32 * ks, lane);
            rl[ks] = frag<LDL>(sRTl, 0, 32 * ks, lane);
        }
        if constexpr (!SEGP) {
            f32x4 o2 = zero4();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks <= wave / 2) {   // MTb is lower triangular
                    const bf16x8 mh = as_bf16x8(mc[ks][0]), ml = as_bf16x8(mc[ks][1]);
                    o2 = mfma16(ml, rh[ks], o2);
                    o2 = mfma16(mh, rl[ks], o2);
                    o2 = mfma16(mh, rh[ks], o2);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) so[(4 * g + r) * LDO + c16] = p.scale * (o1[r] + o2[r]);
        }
#pragma unroll
        for (int s2 = 0; s2 < STW; ++s2) {
            f32x4 ds = zero4();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 wh = as_bf16x8(wc[s2][ks][0]), wl = as_bf16x8(wc[s2][ks][1]);
                ds = mfma16(wl, rh[ks], ds);
                ds = mfma16(wh, rl[ks], ds);
                ds = mfma16(wh, rh[ks], ds);
            }
            if constexpr (DECAY) {
#pragma unroll
                for (int r = 0; r < 4; ++r) S[s2][r] = __builtin_fmaf(S[s2][r], ec[s2][r], ds[r]);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) S[s2][r] += ds[r];
            }
        }
        write_state_lds();
        if constexpr (VEC) prestore(so_n, sp_n);   // the next chunk's tiles (SPLIT: the V tile only)
    };
    for (int c = c_begin; c < c_end; c += 2) {
        step(c, wcur, ecur, mcur, wnxt, enxt, mnxt);
        if (c + 1 < c_end) step(c + 1, wnxt, enxt, mnxt, wcur, ecur, mcur);
    }
    if (!SEGP) store_outputs(static_cast<int64_t>(c_end - 1) * L);
    if constexpr (VEC && DECAY) {
#pragma unroll
        for (int i = 0; i < NTOUCH; ++i) l2sink |= l2x[i];
        asm volatile("" ::"v"(l2sink));   // the touches stay
    }
    // the state leaving the segment: s_final (last segment), the state entering
    // segment 1 (segment pass, segment 0), or columns of A_s | B_s
    float* sout = nullptr;
    int64_t ld = V, col = v0 + c16;
    bool colok = col < V;
    if (!SEGP) {
        if (seg == p.nseg - 1) sout = p.s_final + (static_cast<int64_t>(b) * H + h) * K * V;
    } else if (seg == 0) {
        sout = p.seg_state + (static_cast<int64_t>(p.B) * H + bh) * K * V;   // segment 1's entering state
    } else {
        sout = p.seg_ab + (static_cast<int64_t>(seg) * p.B * H + bh) * K * (K + V);
        ld = K + V;
        col = atile ? 16 * vt + c16 : K + v0 + c16;
        colok = atile ? 16 * vt + c16 < K : v0 + c16 < V;
    }
    if (sout) {
#pragma unroll
        for (int s2 = 0; s2 < STW; ++s2) {
            const int sr = STW * wave + s2;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 16 * sr + 4 * g + r;
                if (d < K && colok) sout[d * ld + col] = S[s2][r];
            }
        }
    }
}

// The states entering segments 2 .. nseg - 1, one after another:
// S_{s+1} = A_s S_s + B_s, in fp32; a workgroup owns a 16-column V-tile of
// one (batch, head) (its columns depend on no other columns).  The chain over
// segments is sequential, so each step is kept short: A_s comes into LDS from
// 16-byte pieces loaded one step ahead (the loads do not depend on the chain),
// and the product runs on the fp32 matrix cores (16x16x4: lane l holds
// A[l % 16][l / 16], B[l / 16][l % 16] and C[4 (l / 16) + r][l % 16]), wave w
// owning the 16-row tiles w, w + 4, ... (KP / 64 of them).  Four consecutive keys of a
// lane's row feed four products in turn (the contraction index permuted the
// same way in A and B), so one 16-byte LDS read serves four products.  Rows
// and keys past K are zero.
template <int KP>
__global__ __launch_bounds__(NT) void delta_seg_prefix_kernel(DeltaArgs p) {
    constexpr int LDA = KP + 4;            // 16-byte aligned rows, 4 banks apart
    constexpr int NP = KP * KP / 4 / NT;   // 16-byte pieces of A_s per thread
    constexpr int RT = KP / 64;            // 16-row tiles per wave
    static_assert(NT == 256 && VT == 16, "four waves, 16-column tiles");
    __shared__ __align__(16) float sST[VT * LDA];   // S_s^T: [column][key]
    __shared__ __align__(16) float sA[KP * LDA];    // A_s: [row][key]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int vt = blockIdx.x % p.vtiles, bh = blockIdx.x / p.vtiles;
    const int K = p.K, V = p.V;
    const int64_t bhs = static_cast<int64_t>(p.B) * p.H;
    const int col = VT * vt + c16;
    // 16-byte loads when every row of A_s | B_s starts 16-byte aligned
    const bool v4 = (K + V) % 4 == 0 && reinterpret_cast<uintptr_t>(p.seg_ab) % 16 == 0;
    f32x4 pa[NP];
    auto load_a = [&](int s) {
        const float* ab = p.seg_ab + (s * bhs + bh) * K * (K + V);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int pc = tid + j * NT, r = pc / (KP / 4), e0 = (pc % (KP / 4)) * 4;
            const float* src = ab + static_cast<int64_t>(r) * (K + V) + e0;
            // (no use of the loaded values here: a use would wait for each load
            // in turn; keys past K - 1 are zeroed where the pieces are stored)
            f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
            if (r < K && e0 < K) {
                if (v4) {
                    x = *reinterpret_cast<const f32x4*>(src);   // may run past key K - 1 into B_s
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (e0 + q < K) x[q] = src[q];
                }
            }
            pa[j] = x;
        }
    };
    for (int i = tid; i < KP * VT; i += NT) {
        const int e = i / VT, c = i % VT;
        sST[c * LDA + e] = e < K && VT * vt + c < V
                               ? p.seg_state[(bhs + bh) * K * V + static_cast<int64_t>(e) * V + VT * vt + c]
                               : 0.0f;
    }
    if (p.nseg > 2) load_a(1);
    for (int s = 1; s <= p.nseg - 2; ++s) {
        const float* ab = p.seg_ab + (s * bhs + bh) * K * (K + V);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int pc = tid + j * NT, r = pc / (KP / 4), e0 = (pc % (KP / 4)) * 4;
            f32x4 x = pa[j];
            if (e0 + 4 > K) {
#pragma unroll
                for (int q = 0; q < 4; ++q) x[q] = e0 + q < K ? x[q] : 0.0f;
            }
            *reinterpret_cast<f32x4*>(sA + r * LDA + e0) = x;
        }
        // B_s into the accumulators: rows 16 (wave + 4 t) + 4 g + r, column col
        f32x4 acc[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 16 * (wave + 4 * t) + 4 * g + r;
                acc[t][r] = d < K && col < V ? ab[static_cast<int64_t>(d) * (K + V) + K + col] : 0.0f;
            }
        __syncthreads();   // A_s staged, S_s written
        if (s + 1 <= p.nseg - 2) load_a(s + 1);   // in flight during the product
#pragma unroll
        for (int kb = 0; kb < KP / 16; ++kb) {
            const f32x4 b4 = *reinterpret_cast<const f32x4*>(sST + c16 * LDA + 16 * kb + 4 * g);
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                const f32x4 a4 = *reinterpret_cast<const f32x4*>(sA + (16 * (wave + 4 * t) + c16) * LDA + 16 * kb + 4 * g);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[j], b4[j], acc[t], 0, 0, 0);
            }
        }
        __syncthreads();   // every read of S_s and A_s is done
        float* out = p.seg_state + ((s + 1) * bhs + bh) * K * V;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int d0 = 16 * (wave + 4 * t) + 4 * g;
            *reinterpret_cast<f32x4*>(sST + c16 * LDA + d0) = acc[t];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (d0 + r < K && col < V) out[static_cast<int64_t>(d0 + r) * V + col] = acc[t][r];
        }
    }
}

template <int KP, bool DECAY, bool VEC>
void launch_passes(const DeltaArgs& a, hipStream_t stream) {
    const int64_t gprep = static_cast<int64_t>(a.B) * a.H * a.nchunks;
    const int64_t units = static_cast<int64_t>(a.B) * a.H * a.vtiles;
    hipLaunchKernelGGL((delta_prep_kernel<KP, VEC, DECAY>), dim3(static_cast<unsigned>(gprep)), dim3(NT), 0, stream,
                       a);
    if (a.nseg > 1) {
        const int kt = (a.K + VT - 1) / VT;
        const int64_t gseg = static_cast<int64_t>(a.B) * a.H * (a.vtiles + (a.nseg - 2) * (kt + a.vtiles));
        hipLaunchKernelGGL((delta_scan_kernel<KP, VEC, DECAY, true>), dim3(static_cast<unsigned>(gseg)), dim3(NT), 0,
                           stream, a);
        if (a.nseg > 2)
            hipLaunchKernelGGL((delta_seg_prefix_kernel<KP>), dim3(static_cast<unsigned>(units)), dim3(NT), 0, stream,
                               a);
    }
    hipLaunchKernelGGL((delta_scan_kernel<KP, VEC, DECAY>), dim3(static_cast<unsigned>(units * a.nseg)), dim3(NT), 0,
                       stream, a);
}

template <int KP, bool DECAY>
hipError_t launch_t(const DeltaArgs& a, bool vec, hipStream_t stream) {
    if (vec) launch_passes<KP, DECAY, true>(a, stream);
    else launch_passes<KP, DECAY, false>(a, stream);
    return hipGetLastError();
}

}  // namespace

int delta_vtile() { return VT; }

size_t delta_chunk_workspace_bytes(int B, int T, int H, int K, bool decay) {
    const int64_t nchunks = (static_cast<int64_t>(T) + L - 1) / L;
    const size_t per_chunk = decay ? (K <= 64 ? chunk_u16<64, true>() : chunk_u16<128, true>())
                                   : (K <= 64 ? chunk_u16<64, false>() : chunk_u16<128, false>());
    return static_cast<size_t>(B) * H * nchunks * per_chunk * sizeof(u16);
}

size_t delta_workspace_bytes(int B, int T, int H, int K, int V, bool decay, int nseg) {
    size_t n = delta_chunk_workspace_bytes(B, T, H, K, decay);
    if (nseg > 1) {
        const size_t bh = static_cast<size_t>(B) * H;
        n += static_cast<size_t>(nseg) * bh * K * V * sizeof(float);          // seg_state
        n += static_cast<size_t>(nseg) * bh * K * (K + V) * sizeof(float);    // seg_ab
    }
    return n;
}

// Time segments: where the (batch, head, V-tile) workgroups leave most compute
// units idle, split the chunks into the most segments whose output pass and
// segment pass (which also runs ceil(K / 16) identity tiles per inner
// segment) each fit the compute units once, with at least 8 chunks a segment.
int delta_plan_segments(int B, int T, int H, int K, int V, int num_cus, int requested) {
    const int64_t nchunks = (static_cast<int64_t>(T) + L - 1) / L;
    if (requested > 0) return static_cast<int>(requested < nchunks ? requested : nchunks);
    const int64_t vtiles = (V + VT - 1) / VT, kt = (K + VT - 1) / VT;
    const int64_t units = static_cast<int64_t>(B) * H * vtiles;
    int best = 1;
    for (int ns = 2; ns <= 64; ++ns) {
        const int64_t cps = (nchunks + ns - 1) / ns;
        if (cps < 8 || (nchunks + cps - 1) / cps != ns) continue;
        if (units * ns > num_cus) break;
        if (static_cast<int64_t>(B) * H * (vtiles + (ns - 2) * (kt + vtiles)) > num_cus) break;
        best = ns;
    }
    return best;
}

int delta_decay_max_k() { return KD; }

hipError_t launch_scan_delta(const DeltaParams& prm, void* workspace, hipStream_t stream) {
    DeltaArgs a{};
    a.q = reinterpret_cast<const u16*>(prm.q);
    a.k = reinterpret_cast<const u16*>(prm.k);
    a.v = reinterpret_cast<const u16*>(prm.v);
    a.beta = prm.beta;
    a.g = prm.g;
    a.s0 = prm.s0;
    a.o = prm.o;
    a.s_final = prm.s_final;
    a.ws = static_cast<u16*>(workspace);
    a.B = prm.B;
    a.T = prm.T;
    a.H = prm.H;
    a.K = prm.K;
    a.V = prm.V;
    a.scale = prm.scale;
    a.vtiles = (prm.V + VT - 1) / VT;
    a.nchunks = (prm.T + L - 1) / L;
    a.out_bf16 = prm.out_bf16;
    a.nseg = prm.nseg > 1 ? prm.nseg : 1;
    a.cps = (a.nchunks + a.nseg - 1) / a.nseg;
    a.nseg = (a.nchunks + a.cps - 1) / a.cps;   // no empty segment
    if (a.nseg > 1) {
        const bool decay = prm.g != nullptr;
        char* base = static_cast<char*>(workspace) + delta_chunk_workspace_bytes(prm.B, prm.T, prm.H, prm.K, decay);
        a.seg_state = reinterpret_cast<float*>(base);
        a.seg_ab = a.seg_state + static_cast<size_t>(a.nseg) * prm.B * prm.H * prm.K * prm.V;
    }
    if (prm.g) {
        if (prm.K > KD) return hipErrorInvalidValue;
        return prm.K <= 64 ? launch_t<64, true>(a, prm.vec != 0, stream) : launch_t<128, true>(a, prm.vec != 0, stream);
    }
    return prm.K <= 64 ? launch_t<64, false>(a, prm.vec != 0, stream) : launch_t<128, false>(a, prm.vec != 0, stream);
}

}  // namespace lrs

