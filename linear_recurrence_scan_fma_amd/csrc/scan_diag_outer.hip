// Decay-separable outer-product state scan with readout, on gfx950 matrix cores:
//
//   S_t[i][j] = exp(g_t[i]) S_{t-1}[i][j] + kappa_t k_t[i] v_t[j]
//   o_t[j]    = scale * sum_i S_t[i][j] q_t[i]
//
// Mamba-2 (one log-decay dt*A per head and step, injection dt*B, readout C)
// and GLA (per-key log-decay gk, readout scale S^T q) [SunnyNet log §4.1, §4.3:
// "SunnyNet 工程化实录：一个 O(N) 架构如何长出自己的 C 推理运行时",
// developer.aliyun.com/article/1773847; restated in the llama.cpp comparison
// "我拿同一份权重和 llama.cpp 正面比了一场：我手写的 C 内核，慢了 1.1–1.7 倍" §3].
//
// Chunked form (chunk of L = 64 steps, state S0 entering the chunk, G_t the
// within-chunk cumulative log-decay including step t, G_L its last value):
//   o_t = scale * ( sum_{tau<=t} P[t][tau] v_tau + sum_d q_t[d] e^{G_t[d]} S0[d][:] )
//   P[t][tau] = kappa_tau sum_d q_t[d] k_tau[d] e^{G_t[d] - G_tau[d]}
//   S_L = diag(e^{G_L}) S0 + sum_tau diag(e^{G_L - G_tau}) kappa_tau k_tau v_tau^T
// which is the sequential recurrence regrouped (no approximation).  Across
// chunks the state obeys S <- a (.) S + U with a diagonal `a`, so the time
// axis also splits into segments: a first kernel reduces each segment to its
// pair (a_seg, U_seg) from a zero state (the first segment from S0), a prefix
// kernel turns the pairs into the state after each segment, and the output
// kernel starts each segment from the state after the one before it.
//
// Work split: a workgroup owns (batch, head, 64-column V-tile, segment); wave w
// owns state columns 16w..16w+15 for all keys, as 16x16 fp32 accumulator tiles
// held in registers for the whole segment.  Per chunk the raw inputs go to LDS
// row-major (prefetched into registers during the previous chunk), then:
//   scores  P^T = K Q^T on v_mfma_f32_16x16x32_bf16, masked and scaled, to LDS;
//   readout O^T = S^T Q^T (the state tiles are the left operand in place) plus
//           V^T P^T, with V^T and K^T taken by the transposing LDS read;
//   update  S = a (.) S + K~^T V~.
// With the contraction slots of mfma_util.h (lane group g holds {4g..4g+3} u
// {16+4g..16+4g+3} of each 32-wide step), two accumulator tiles are exactly a
// left operand, so the state never leaves its registers.
//
// Precision: q, k, v are bf16 and enter the matrix cores exactly; fp32 operands
// (the state, P, decay-scaled keys or values) are split into hi + lo bf16 terms.
//  * scalar decay (mode 0): P = (K Q^T) scaled pair by pair by
//    kappa_tau e^{G_t - G_tau}; the readout is scaled by e^{G_t} per row; the
//    update weight kappa_tau e^{G_L - G_tau} goes on the values.  Stable for any
//    decay strength.
//  * per-key decay (mode 1): q~ = q o e^{G_t - G_L} and k~ = kappa k o e^{G_L - G_t}
//    give P = q~ k~^T, readout q~ (e^{G_L} o S0), update k~^T v.  Both factors stay
//    inside the fp32/bf16 range while the chunk's decay is below 60 nats on every
//    key (GLA-shaped gates use a few nats); otherwise the chunk evaluates P pair
//    by pair with exact exponentials and reads out with q o e^{G_t} and S0.
#include <atomic>

#include "lrs_internal.h"
#include "mfma_util.h"

namespace lrs {
namespace {

constexpr int L = 64;     // chunk length
// A workgroup has WPB waves (4 or 8); wave w owns 16 state columns, so a
// workgroup covers a V-tile of 16 WPB columns.  Heads wider than 64 columns use
// 8 waves, so that the per-chunk staging and scores are shared by all columns.
inline int waves_for(int V) { return V > 64 ? 8 : 4; }
constexpr int kMinChunksPerSegment = 4;
constexpr float kFastPathMaxDecay = 60.0f;

struct DiagArgs {
    const u16* q;
    const u16* k;
    const u16* v;
    const float* g;
    const float* ks;
    const float* s0;
    float* o;
    float* s_final;
    float* agg_u;    // [nseg-1][unit][wave][KP/16][lane][4]: per segment, its state from zero
                     // (from s0 for the first), then in place the state after it; in the
                     // accumulator-tile order of the lanes that own them
    float* agg_a;    // [nseg-1][B*H][KP]: segment decay products (1 past K)
    int B, T, H, Hg, K, V;
    float scale;
    int vtiles;
    int nchunks, nseg, cps;   // chunks, segments, chunks per segment
    // output epilogue (EPI variants): kind 0 none, 1 o + D_h v, 2 RMSNorm(o) w silu(z)
    int epi_kind;
    int out_bf16;             // o is bf16 (else fp32)
    const float* d_skip;      // [H]
    const u16* gate;          // z, bf16 [B,T,H,V]
    const float* norm_w;      // [V], nullable (ones)
    float eps;
};

__device__ __forceinline__ void store4(u16* dst, const u16 (&x)[4]) {
    u32x2 w = {x[0] | (static_cast<uint32_t>(x[1]) << 16), x[2] | (static_cast<uint32_t>(x[3]) << 16)};
    *reinterpret_cast<u32x2*>(dst) = w;
}

__device__ __forceinline__ u16 half_elem(const u32x2& v, int e) {
    const uint32_t w = e < 2 ? v.x : v.y;
    return static_cast<u16>((e & 1) ? (w >> 16) : (w & 0xffff));
}

// Score blocks (key block, query block), key block <= query block, per wave:
// {(0,0),(0,1),(0,2)}, {(1,1),(1,2),(1,3)}, {(2,2),(2,3)}, {(0,3),(3,3)}.
__device__ __forceinline__ bool score_job(int wave, int n, int& kb, int& qb) {
    switch (wave * 3 + n) {
        case 0: kb = 0; qb = 0; return true;
        case 1: kb = 0; qb = 1; return true;
        case 2: kb = 0; qb = 2; return true;
        case 3: kb = 1; qb = 1; return true;
        case 4: kb = 1; qb = 2; return true;
        case 5: kb = 1; qb = 3; return true;
        case 6: kb = 2; qb = 2; return true;
        case 7: kb = 2; qb = 3; return true;
        case 9: kb = 0; qb = 3; return true;
        case 10: kb = 3; qb = 3; return true;
        default: return false;
    }
}

// Score blocks with 8 waves: block wave (and wave + 8) of the list
// (0,0),(0,1),(0,2),(0,3),(1,1),(1,2),(1,3),(2,2),(2,3),(3,3).
__device__ __forceinline__ bool score_job8(int wave, int n, int& kb, int& qb) {
    const int idx = wave + 8 * n;
    if (idx >= 10) return false;
    kb = idx < 4 ? 0 : (idx < 7 ? 1 : (idx < 9 ? 2 : 3));
    const int first = kb == 0 ? 0 : (kb == 1 ? 4 : (kb == 2 ? 7 : 9));
    qb = kb + (idx - first);
    return true;
}

// AGG = true: segment reduction (a_seg, U_seg) from a zero state, no outputs.
// AGG = false: outputs and the final state, starting from the state entering the segment.
// KK = true (per-key decay only): kappa per key, k_scale [B,T,H,K].
// EPI = true (output pass only): the output epilogue and dtype of DiagArgs.
template <int MODE, int KP, int WPB, bool VEC, bool AGG, bool KK = false, bool EPI = false>
__global__ __launch_bounds__(64 * WPB) void diag_outer_kernel(DiagArgs p) {
    static_assert(!KK || MODE == 1, "a per-key kappa needs the per-key decay path");
    static_assert(!(EPI && AGG), "the epilogue belongs to the output pass");
    constexpr bool OUT = !AGG;
    constexpr int NT = 64 * WPB;   // threads per workgroup
    constexpr int VT = 16 * WPB;   // V-tile width
    // LDS row strides (bf16 elements), chosen by the reads each array serves
    // (LDS: 32 four-byte banks; an 8-byte read serves 16 lanes per pass, a
    // transposing read 16 lanes from 4 rows):
    //  * K and V feed the transposing reads of the update and the readout:
    //    rows 2 KP + 32 (2 VT + 32) bytes apart put 4 consecutive rows on
    //    disjoint 8-bank groups;
    //  * Q and P feed 8-byte reads of 16 consecutive rows at one column
    //    (readout operands, and the scores' Q operand): rows 8 bytes off a
    //    multiple of 128 put those 16 reads on disjoint bank pairs.  Q rows are
    //    then 8-byte aligned only, so Q is written and read in 8-byte pieces.
    constexpr int LDK = KP + 16;
    constexpr int LDV = VT + 16;
    constexpr int LDQ = KP + 4;
    constexpr int LDP = L + 4;
    constexpr int KB = KP / 16;   // 16-row state tiles per wave
    constexpr int KM = KP / 32;   // 32-wide steps over the key axis
    constexpr int NPL = MODE == 1 ? 2 : 1;   // hi/lo planes of the q/k operands
    constexpr int PQ = L * KP / 8 / NT;      // mode 0: 16-byte q/k pieces per thread
    constexpr int PV = L * VT / 8 / NT;      // 16-byte v pieces per thread
    constexpr int KG = KP / 4;               // mode 1: threads per row (4 keys each)
    constexpr int RG = NT / KG;              // mode 1: row groups
    constexpr int RPG = L / RG;              // mode 1: rows per thread
    constexpr int NQ = MODE == 0 ? PQ : RPG;
    static_assert(PQ >= 1 && PV >= 1 && RPG >= 1, "tile shape");
    static_assert(MODE == 0 || NPL * L * LDK * 2 >= L * KP * 4, "fallback scores reuse the key operand space");
    static_assert((2 * LDK) % 16 == 0 && (2 * LDV) % 16 == 0 && (2 * LDQ) % 8 == 0 && (2 * LDP) % 8 == 0, "row alignment");

    __shared__ __align__(16) u16 sQ[OUT ? NPL * L * LDQ : 8];
    __shared__ __align__(16) u16 sK[NPL * L * LDK];
    __shared__ __align__(16) u16 sV[L * LDV];
    __shared__ __align__(16) u16 sP[OUT ? 2 * L * LDP : 8];
    __shared__ __align__(16) float sG[MODE == 0 ? L : 1];      // cumulative log decay
    __shared__ float sEG[MODE == 0 ? L : 1];     // scale e^{G_t}
    __shared__ __align__(16) float sW[MODE == 0 ? L : 1];   // kappa_t e^{G_L - G_t}
    __shared__ __align__(16) float sKap[L];                    // scale kappa_t (scores)
    __shared__ float sDec[1];                    // mode 0: e^{G_L}
    __shared__ __align__(16) float sTot[MODE == 1 ? RG * KP : 1];
    __shared__ float sGL[MODE == 1 ? KP : 1];    // G_L per key
    __shared__ __align__(16) float sEGL[MODE == 1 ? KP : 1];   // e^{G_L} per key
    __shared__ float sRS[EPI ? WPB * L : 1];   // epilogue: per-wave sums of squares of each step's row
    __shared__ __align__(16) float sNW[EPI ? 16 * WPB : 1];   // epilogue: RMSNorm weight of the tile's columns

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int g4 = lane >> 4;
    const int c16 = lane & 15;
    const int nsegk = AGG ? p.nseg - 1 : p.nseg;
    const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
    const int seg = lid % nsegk;
    const int rest = lid / nsegk;
    const int vt = rest % p.vtiles;
    const int bh = rest / p.vtiles;
    const int b = bh / p.H;
    const int h = bh - b * p.H;
    const int grp = h / (p.H / p.Hg);
    const int v0 = vt * VT;
    const int64_t T = p.T;
    const int K = p.K, V = p.V, H = p.H, Hg = p.Hg;
    const int c_begin = seg * p.cps;
    const int c_end = min(c_begin + p.cps, p.nchunks);
    const int jcol = v0 + 16 * wave + c16;   // this lane's state column
    const float scale = p.scale;

    // Batch-row bases and byte sizes; each chunk reads through a window that
    // starts at its first step (vector path), so per-lane offsets are fixed.
    const int64_t qk_row = static_cast<int64_t>(Hg) * K * 2;        // bytes per step
    const int64_t v_row = static_cast<int64_t>(H) * V * 2;
    const int64_t g_row = static_cast<int64_t>(H) * (MODE == 1 ? K : 1) * 4;
    const int64_t s_row = static_cast<int64_t>(H) * (KK ? K : 1) * 4;   // k_scale
    const int64_t o_row = static_cast<int64_t>(H) * V * 4;
    const u16* qb = p.q + b * T * Hg * static_cast<int64_t>(K);
    const u16* kb_ = p.k + b * T * Hg * static_cast<int64_t>(K);
    const u16* vb = p.v + b * T * H * static_cast<int64_t>(V);
    const float* gb = p.g + b * T * H * static_cast<int64_t>(MODE == 1 ? K : 1);
    const float* ksb = p.ks ? p.ks + b * T * H * static_cast<int64_t>(KK ? K : 1) : nullptr;
    float* ob = p.o + b * T * H * static_cast<int64_t>(V);

    // per-lane offsets within a chunk window
    int offq[NQ], offg[MODE == 1 ? NQ : 1], offs[MODE == 1 ? NQ : 1], offv[PV];
    if constexpr (MODE == 0) {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int pi = tid + NT * i, row = pi / (KP / 8), c8 = (pi % (KP / 8)) * 8;
            offq[i] = c8 < K ? ((row * Hg + grp) * K + c8) * 2 : kBufOOB;
        }
        offg[0] = (tid * H + h) * 4;
    } else {
        const int kg = tid % KG, rg = tid / KG, d0 = kg * 4;
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            const int t = rg * RPG + r;
            offq[r] = d0 < K ? ((t * Hg + grp) * K + d0) * 2 : kBufOOB;
            offg[r] = d0 < K ? ((t * H + h) * K + d0) * 4 : kBufOOB;
            offs[r] = (t * H + h) * 4;
        }
    }
#pragma unroll
    for (int i = 0; i < PV; ++i) {
        const int pi = tid + NT * i, row = pi / (VT / 8), c8 = (pi % (VT / 8)) * 8;
        offv[i] = v0 + c8 < V ? ((row * H + h) * V + v0 + c8) * 2 : kBufOOB;
    }
    const int offo = jcol - c16 + 4 * g4 < V ? ((c16 * H + h) * V + v0 + 16 * wave + 4 * g4) * 4 : kBufOOB;
    // epilogue: bf16 views of the gate and of the output (same [B,T,H,V] layout)
    const int off2 = offo == kBufOOB ? kBufOOB : offo / 2;
    const int64_t z_row = static_cast<int64_t>(H) * V * 2;
    const u16* zb = EPI && p.gate ? p.gate + b * T * H * static_cast<int64_t>(V) : nullptr;
    u16* ob16 = reinterpret_cast<u16*>(p.o) + b * T * H * static_cast<int64_t>(V);
    float dsk = 0.0f;
    if constexpr (EPI) {
        // RMSNorm weight of the tile's columns (read after the first chunk's barriers)
        if (tid < VT) sNW[tid] = (p.norm_w && v0 + tid < V) ? p.norm_w[v0 + tid] : 1.0f;
        if (p.d_skip) dsk = p.d_skip[h];
    }

    // ---- prefetch registers: raw inputs of one chunk ----
    // mode 0: q/k as 16-byte row pieces; mode 1: 4 keys x RPG rows per thread
    u32x4 cq[MODE == 0 ? NQ : 1], ck[MODE == 0 ? NQ : 1];
    u32x2 cq2[MODE == 1 ? NQ : 1], ck2[MODE == 1 ? NQ : 1];
    u32x4 cgv[MODE == 1 ? NQ : 1];
    float ckp[MODE == 1 ? NQ : 1];
    u32x4 ckk[KK ? NQ : 1];   // per-key kappa, 4 keys per row, as g
    u32x4 cv[PV];
    float cgs = 0.0f, ckap = 0.0f;

    // part 0: q, k; part 1: v, g, kappa (vector path; the scalar path loads
    // everything in part 0).  Two short bursts issued after two different
    // barriers keep the memory queue from stalling a wave behind one long one.
    auto load_chunk = [&](int c, int part) {
        const int64_t t0 = static_cast<int64_t>(c) * L;
        if constexpr (VEC) {
            const BufRes wq = make_rsrc_window(qb, T * qk_row, t0 * qk_row);
            const BufRes wk = make_rsrc_window(kb_, T * qk_row, t0 * qk_row);
            const BufRes wv = make_rsrc_window(vb, T * v_row, t0 * v_row);
            const BufRes wg = make_rsrc_window(gb, T * g_row, t0 * g_row);
            const BufRes ws = make_rsrc_window(ksb ? static_cast<const void*>(ksb) : gb, ksb ? T * s_row : 0,
                                               t0 * s_row);
            if (part == 0) {
                if constexpr (MODE == 0) {
#pragma unroll
                    for (int i = 0; i < NQ; ++i) {
                        if constexpr (OUT) cq[i] = buf_load16(wq, offq[i]);
                        ck[i] = buf_load16(wk, offq[i]);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < NQ; ++r) {
                        if constexpr (OUT) cq2[r] = __builtin_amdgcn_raw_buffer_load_b64(wq, offq[r], 0, 0);
                        ck2[r] = __builtin_amdgcn_raw_buffer_load_b64(wk, offq[r], 0, 0);
                    }
                }
            } else {
                if constexpr (MODE == 0) {
                    if (tid < L) {
                        cgs = buf_load_f32(wg, offg[0]);
                        ckap = buf_load_f32(ws, offg[0]);   // raw; NULL k_scale handled at use
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < NQ; ++r) {
                        cgv[r] = buf_load16(wg, offg[r]);
                        if constexpr (KK) ckk[r] = buf_load16(ws, offg[r]);
                        else ckp[r] = buf_load_f32(ws, offs[r]);   // raw; NULL k_scale handled at use
                    }
                }
#pragma unroll
                for (int i = 0; i < PV; ++i) cv[i] = buf_load16(wv, offv[i]);
            }
        } else if (part == 0) {
            if constexpr (MODE == 0) {
#pragma unroll
                for (int i = 0; i < NQ; ++i) {
                    const int pi = tid + NT * i, row = pi / (KP / 8), c8 = (pi % (KP / 8)) * 8;
                    const int64_t t = t0 + row;
                    cq[i] = u32x4{0u, 0u, 0u, 0u};
                    ck[i] = u32x4{0u, 0u, 0u, 0u};
                    if (t < T) {
                        const int64_t off = (t * Hg + grp) * static_cast<int64_t>(K);
                        if constexpr (OUT) cq[i] = load8_bf16(qb + off, c8, K, false);
                        ck[i] = load8_bf16(kb_ + off, c8, K, false);
                    }
                }
                if (tid < L) {
                    const int64_t t = t0 + tid;
                    cgs = 0.0f;
                    ckap = 0.0f;
                    if (t < T) {
                        cgs = gb[t * H + h];
                        ckap = ksb ? ksb[t * H + h] : 1.0f;
                    }
                }
            } else {
                const int kg = tid % KG, rg = tid / KG, d0 = kg * 4;
#pragma unroll
                for (int r = 0; r < NQ; ++r) {
                    const int64_t t = t0 + rg * RPG + r;
                    u16 qe[4] = {0, 0, 0, 0}, ke[4] = {0, 0, 0, 0};
                    float ge[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                    float kk4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                    float kp = 0.0f;
                    if (t < T) {
                        const int64_t oq = (t * Hg + grp) * static_cast<int64_t>(K);
                        const int64_t og = (t * H + h) * static_cast<int64_t>(K);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (d0 + e < K) {
                                if constexpr (OUT) qe[e] = qb[oq + d0 + e];
                                ke[e] = kb_[oq + d0 + e];
                                ge[e] = gb[og + d0 + e];
                                if constexpr (KK) kk4[e] = ksb[og + d0 + e];
                            }
                        }
                        if constexpr (!KK) kp = ksb ? ksb[t * H + h] : 1.0f;
                    }
                    if constexpr (KK)
                        ckk[r] = u32x4{__float_as_uint(kk4[0]), __float_as_uint(kk4[1]), __float_as_uint(kk4[2]),
                                       __float_as_uint(kk4[3])};
                    cq2[r] = u32x2{qe[0] | (static_cast<uint32_t>(qe[1]) << 16),
                                   qe[2] | (static_cast<uint32_t>(qe[3]) << 16)};
                    ck2[r] = u32x2{ke[0] | (static_cast<uint32_t>(ke[1]) << 16),
                                   ke[2] | (static_cast<uint32_t>(ke[3]) << 16)};
                    cgv[r] = u32x4{__float_as_uint(ge[0]), __float_as_uint(ge[1]), __float_as_uint(ge[2]),
                                   __float_as_uint(ge[3])};
                    ckp[r] = kp;
                }
            }
#pragma unroll
            for (int i = 0; i < PV; ++i) {
                const int pi = tid + NT * i, row = pi / (VT / 8), c8 = (pi % (VT / 8)) * 8;
                const int64_t t = t0 + row;
                cv[i] = u32x4{0u, 0u, 0u, 0u};
                if (t < T) cv[i] = load8_bf16(vb + (t * H + h) * static_cast<int64_t>(V) + v0, c8, V - v0, false);
            }
        }
    };

    // ---- state entering the segment: s0 for the first, else the prefix state
    // that the segment pass and the prefix kernel left for the segment before ----
    const int units = p.B * H * p.vtiles;
    f32x4 S[KB];
    if (OUT && seg > 0) {
        const float* ub = p.agg_u + ((static_cast<int64_t>(seg - 1) * units + rest) * WPB + wave) * (KB * 256);
#pragma unroll
        for (int db = 0; db < KB; ++db) S[db] = *reinterpret_cast<const f32x4*>(ub + (db * 64 + lane) * 4);
    } else {
#pragma unroll
        for (int db = 0; db < KB; ++db) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 16 * db + 4 * g4 + r;
                float x = 0.0f;
                if (seg == 0 && p.s0 && d < K && jcol < V) x = p.s0[((static_cast<int64_t>(b) * H + h) * K + d) * V + jcol];
                S[db][r] = x;
            }
        }
    }
    if constexpr (OUT) {
        // score blocks right of the diagonal that the readout reads: always zero
        if (tid < 256) {
            const int blk = tid >> 7, plane = (tid >> 6) & 1, row = (tid >> 2) & 15, quad = tid & 3;
            const int t = 32 * blk + row, c0 = 32 * blk + 16 + 4 * quad;
            const u16 z[4] = {0, 0, 0, 0};
            store4(sP + plane * L * LDP + t * LDP + c0, z);
        }
    }
    float lsum = 0.0f;   // segment log-decay (mode 0: uniform; mode 1: key `tid`)

    if (c_begin < c_end) {
        load_chunk(c_begin, 0);
        load_chunk(c_begin, 1);
    }

    for (int c = c_begin; c < c_end; ++c) {
        const int64_t t0 = static_cast<int64_t>(c) * L;
        bool fast = true;

        // ---- stage: raw or decay-scaled operands into LDS ----
#pragma unroll
        for (int i = 0; i < PV; ++i) {
            const int pi = tid + NT * i;
            *reinterpret_cast<u32x4*>(sV + (pi / (VT / 8)) * LDV + (pi % (VT / 8)) * 8) = cv[i];
        }
        if constexpr (MODE == 0) {
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int pi = tid + NT * i;
                const int row = pi / (KP / 8);
                const int c8 = (pi % (KP / 8)) * 8;
                if constexpr (OUT) {
                    // two 8-byte halves; pieces 8..15 of a row write their upper half first,
                    // so the 16 lanes of a pass cover all banks
                    const u32x2 lo2 = {cq[i].x, cq[i].y}, hi2 = {cq[i].z, cq[i].w};
                    const bool swap = ((pi % (KP / 8)) >> 3) & 1;
                    u16* dq = sQ + row * LDQ + c8;
                    *reinterpret_cast<u32x2*>(dq + (swap ? 4 : 0)) = swap ? hi2 : lo2;
                    *reinterpret_cast<u32x2*>(dq + (swap ? 0 : 4)) = swap ? lo2 : hi2;
                }
                *reinterpret_cast<u32x4*>(sK + row * LDK + c8) = ck[i];
            }
            if (wave == 0) {
                float x = cgs;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float y = __shfl_up(x, off);
                    if (lane >= off) x += y;
                }
                const float gl = __shfl(x, 63);
                const float kap = (VEC && !p.ks) ? (t0 + lane < T ? 1.0f : 0.0f) : ckap;
                sG[lane] = x;
                sEG[lane] = scale * __expf(x);
                sW[lane] = kap * __expf(gl - x);
                sKap[lane] = scale * kap;
                if (lane == 0) sDec[0] = __expf(gl);
            }
        } else {
            const int kg = tid % KG, rg = tid / KG, d0 = kg * 4;
            float G[NQ][4];
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int r = 0; r < NQ; ++r) {
                const float ge[4] = {__uint_as_float(cgv[r].x), __uint_as_float(cgv[r].y),
                                     __uint_as_float(cgv[r].z), __uint_as_float(cgv[r].w)};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[e] += ge[e];
                    G[r][e] = acc[e];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sTot[rg * KP + d0 + e] = acc[e];
            __syncthreads();
            float pre[4] = {0.0f, 0.0f, 0.0f, 0.0f}, tot[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int r2 = 0; r2 < RG; ++r2) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(sTot + r2 * KP + d0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (r2 < rg) pre[e] += x[e];
                    tot[e] += x[e];
                }
            }
            bool bad = false;
#pragma unroll
            for (int r = 0; r < NQ; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e) G[r][e] += pre[e];
#pragma unroll
            for (int e = 0; e < 4; ++e) bad = bad || (-tot[e] > kFastPathMaxDecay);
            if constexpr (OUT) fast = !__syncthreads_or(bad);
            if (rg == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sGL[d0 + e] = tot[e];
                    sEGL[d0 + e] = __expf(tot[e]);
                }
            }
            float kapr[NQ];
#pragma unroll
            for (int r = 0; r < NQ; ++r)
                kapr[r] = KK ? 1.0f : (VEC && !p.ks) ? (t0 + rg * RPG + r < T ? 1.0f : 0.0f) : ckp[r];
            // kappa of row r, key d0 + e
            auto kap_at = [&](int r, int e) -> float {
                if constexpr (KK) return __uint_as_float(ckk[r][e]);
                else return kapr[r];
            };
            if (OUT && !fast) {
                // exact scores pair by pair: raw q, k and G into the operand space
                float* sGf = reinterpret_cast<float*>(sK);
#pragma unroll
                for (int r = 0; r < NQ; ++r) {
                    const int t = rg * RPG + r;
                    *reinterpret_cast<u32x2*>(sQ + t * LDQ + d0) = cq2[r];
                    *reinterpret_cast<u32x2*>(sQ + L * LDQ + t * LDQ + d0) = ck2[r];
                    *reinterpret_cast<f32x4*>(sGf + t * KP + d0) = f32x4{G[r][0], G[r][1], G[r][2], G[r][3]};
                    if (kg == 0) sKap[t] = scale * kapr[r];
                }
                __syncthreads();
                // (the per-key kappa of this rare path is read from memory, so the
                // variant needs no LDS buffer for it)
                for (int idx = tid; idx < L * L; idx += NT) {
                    const int t = idx / L, tau = idx % L;
                    float a = 0.0f;
                    if (tau <= t) {
                        const bool row_ok = t0 + tau < T;
                        const float* kk_row = KK ? ksb + ((t0 + tau) * H + h) * static_cast<int64_t>(K) : nullptr;
                        for (int d = 0; d < KP; ++d) {
                            float kd = bf2f(sQ[L * LDQ + tau * LDQ + d]);
                            if constexpr (KK) kd *= (row_ok && d < K) ? kk_row[d] : 0.0f;
                            a += bf2f(sQ[t * LDQ + d]) * kd * __expf(sGf[t * KP + d] - sGf[tau * KP + d]);
                        }
                        a *= sKap[tau];
                    }
                    u16 hi, lo;
                    split_bf16(a, hi, lo);
                    sP[t * LDP + tau] = hi;
                    sP[L * LDP + t * LDP + tau] = lo;
                }
                __syncthreads();
            }
            // q~ = scale q e^{G_t - G_L} (fallback: scale q e^{G_t}), k~ = kappa k e^{G_L - G_t}
#pragma unroll
            for (int r = 0; r < NQ; ++r) {
                const int t = rg * RPG + r;
                float qv[4], kv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (OUT) qv[e] = bf2f(half_elem(cq2[r], e)) * (scale * __expf(fast ? G[r][e] - tot[e] : G[r][e]));
                    kv[e] = bf2f(half_elem(ck2[r], e)) * (kap_at(r, e) * __expf(tot[e] - G[r][e]));
                }
                uint32_t hq[2], lq[2], hk[2], lk[2];
                if constexpr (OUT) {
                    split2(qv[0], qv[1], hq[0], lq[0]);
                    split2(qv[2], qv[3], hq[1], lq[1]);
                    *reinterpret_cast<u32x2*>(sQ + t * LDQ + d0) = u32x2{hq[0], hq[1]};
                    *reinterpret_cast<u32x2*>(sQ + L * LDQ + t * LDQ + d0) = u32x2{lq[0], lq[1]};
                }
                split2(kv[0], kv[1], hk[0], lk[0]);
                split2(kv[2], kv[3], hk[1], lk[1]);
                *reinterpret_cast<u32x2*>(sK + t * LDK + d0) = u32x2{hk[0], hk[1]};
                *reinterpret_cast<u32x2*>(sK + L * LDK + t * LDK + d0) = u32x2{lk[0], lk[1]};
            }
        }
        __syncthreads();

        // the prefetch registers were consumed by the staging: load the next chunk
        if (c + 1 < c_end) load_chunk(c + 1, 0);
        if constexpr (AGG) {
            if constexpr (MODE == 0) lsum += sG[L - 1];
            else if (tid < KP) lsum += sGL[tid];
        }

        // ---- scores P (key block kb, query block qb) -> LDS as P[t][tau] ----
        if (OUT && fast) {
#pragma unroll
            for (int n = 0; n < (WPB == 4 ? 3 : 2); ++n) {
                int kb, qbk;
                if (!(WPB == 4 ? score_job(wave, n, kb, qbk) : score_job8(wave, n, kb, qbk))) continue;
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < KM; ++ks) {
                    const bf16x8 ah = frag<LDK>(sK, 16 * kb, 32 * ks, lane);
                    const bf16x8 bh_ = frag_b64<LDQ>(sQ, 16 * qbk, 32 * ks, lane);
                    if constexpr (MODE == 1) {
                        const bf16x8 al = frag<LDK>(sK + L * LDK, 16 * kb, 32 * ks, lane);
                        const bf16x8 bl = frag_b64<LDQ>(sQ + L * LDQ, 16 * qbk, 32 * ks, lane);
                        acc = mfma16(al, bh_, acc);
                        acc = mfma16(ah, bl, acc);
                    }
                    acc = mfma16(ah, bh_, acc);
                }
                const int t = 16 * qbk + c16;
                const int tau0 = 16 * kb + 4 * g4;
                float val[4];
                if constexpr (MODE == 0) {
                    const float gt = sG[t];
                    const f32x4 gtau = *reinterpret_cast<const f32x4*>(sG + tau0);
                    const f32x4 ktau = *reinterpret_cast<const f32x4*>(sKap + tau0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float f = ktau[r] * __expf(gt - gtau[r]);   // unused (maybe inf) above the diagonal
                        val[r] = tau0 + r <= t ? acc[r] * f : 0.0f;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) val[r] = tau0 + r <= t ? acc[r] : 0.0f;
                }
                uint32_t hi[2], lo[2];
                split2(val[0], val[1], hi[0], lo[0]);
                split2(val[2], val[3], hi[1], lo[1]);
                *reinterpret_cast<u32x2*>(sP + t * LDP + tau0) = u32x2{hi[0], hi[1]};
                *reinterpret_cast<u32x2*>(sP + L * LDP + t * LDP + tau0) = u32x2{lo[0], lo[1]};
            }
        }
        if constexpr (OUT) __syncthreads();
        if (c + 1 < c_end) load_chunk(c + 1, 1);

        // ---- per wave: readout of its 16 columns and the state update ----
        bf16x8 vA[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) vA[ks] = tr_frag<LDV>(sV, 32 * ks, 16 * wave, lane);

        if constexpr (OUT) {
            // per-key decay reads out from e^{G_L} o S0 (and the update then adds to it)
            if constexpr (MODE == 1) {
                if (fast) {
#pragma unroll
                    for (int db = 0; db < KB; ++db) {
                        const f32x4 a = *reinterpret_cast<const f32x4*>(sEGL + 16 * db + 4 * g4);
                        S[db] *= a;
                    }
                }
            }
            // epilogue gate of this lane's four columns at its four steps (issued before the
            // readout's products, which hide its latency)
            u32x2 zq[EPI ? 4 : 1];
            if constexpr (EPI) {
                if (p.epi_kind == 2) {
                    if constexpr (VEC) {
                        const BufRes wz = make_rsrc_window(zb, T * z_row, t0 * z_row);
#pragma unroll
                        for (int tb = 0; tb < 4; ++tb)
                            zq[tb] = __builtin_amdgcn_raw_buffer_load_b64(
                                wz, off2 == kBufOOB ? kBufOOB : off2 + tb * 16 * static_cast<int>(z_row), 0, 0);
                    } else {
#pragma unroll
                        for (int tb = 0; tb < 4; ++tb) {
                            const int64_t t = t0 + 16 * tb + c16;
                            const int col = v0 + 16 * wave + 4 * g4;
                            u16 z4[4] = {0, 0, 0, 0};
                            if (t < T) {
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    if (col + r < V) z4[r] = zb[(t * H + h) * static_cast<int64_t>(V) + col + r];
                            }
                            zq[tb] = u32x2{z4[0] | (static_cast<uint32_t>(z4[1]) << 16),
                                           z4[2] | (static_cast<uint32_t>(z4[3]) << 16)};
                        }
                    }
                }
            }
            bf16x8 sh[KM], sl[KM];
#pragma unroll
            for (int m = 0; m < KM; ++m) {
                const float x[8] = {S[2 * m][0],     S[2 * m][1],     S[2 * m][2],     S[2 * m][3],
                                    S[2 * m + 1][0], S[2 * m + 1][1], S[2 * m + 1][2], S[2 * m + 1][3]};
                split8(x, sh[m], sl[m]);
            }
            f32x4 acc[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) acc[tb] = zero4();
            // per key step: all four step blocks' operands first, then the products
            // term by term, so that no product waits on the one just issued
#pragma unroll
            for (int m = 0; m < KM; ++m) {
                bf16x8 qh[4], ql[MODE == 1 ? 4 : 1];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const u16* qrow = sQ + (16 * tb + c16) * LDQ + 4 * g4 + 32 * m;
                    qh[tb] = slot_frag(qrow);
                    if constexpr (MODE == 1) ql[tb] = slot_frag(qrow + L * LDQ);
                }
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) acc[tb] = mfma16(sl[m], qh[tb], acc[tb]);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) acc[tb] = mfma16(sh[m], qh[tb], acc[tb]);
                if constexpr (MODE == 1) {
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) acc[tb] = mfma16(sh[m], ql[tb], acc[tb]);
                }
            }
            if constexpr (MODE == 0) {
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) acc[tb] *= sEG[16 * tb + c16];
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int tb = 2 * ks; tb < 4; ++tb) {
                    const u16* prow = sP + (16 * tb + c16) * LDP + 4 * g4 + 32 * ks;
                    acc[tb] = mfma16(vA[ks], slot_frag(prow + L * LDP), acc[tb]);
                    acc[tb] = mfma16(vA[ks], slot_frag(prow), acc[tb]);
                }
            }
            // acc[tb]: rows = columns v0 + 16 wave + 4 g4 + r, column = step t0 + 16 tb + c16
            if constexpr (EPI) {
                if (p.epi_kind == 1) {
                    // skip connection: o + D_h v, v from the chunk's value tile
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) {
                        const u32x2 v4 = *reinterpret_cast<const u32x2*>(sV + (16 * tb + c16) * LDV + 16 * wave + 4 * g4);
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[tb][r] = __builtin_fmaf(dsk, bf2f(half_elem(v4, r)), acc[tb][r]);
                    }
                } else if (p.epi_kind == 2) {
                    // RMSNorm over the value axis (the whole row is in this workgroup), then the gate
                    float ss[4];
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) {
                        float x = 0.0f;
#pragma unroll
                        for (int r = 0; r < 4; ++r) x = __builtin_fmaf(acc[tb][r], acc[tb][r], x);
                        x += __shfl_xor(x, 16);
                        x += __shfl_xor(x, 32);
                        ss[tb] = x;
                    }
                    if (g4 == 0) {
#pragma unroll
                        for (int tb = 0; tb < 4; ++tb) sRS[wave * L + 16 * tb + c16] = ss[tb];
                    }
                    __syncthreads();
                    const float inv_v = 1.0f / static_cast<float>(V);
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) {
                        float tot = 0.0f;
#pragma unroll
                        for (int w = 0; w < WPB; ++w) tot += sRS[w * L + 16 * tb + c16];
                        const float inv = 1.0f / sqrtf(__builtin_fmaf(tot, inv_v, p.eps));
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float z = bf2f(half_elem(zq[tb], r));
                            const float silu = z / (1.0f + __expf(-z));
                            acc[tb][r] = acc[tb][r] * inv * sNW[16 * wave + 4 * g4 + r] * silu;
                        }
                    }
                }
            }
            if (EPI && p.out_bf16) {
                // bf16 output, rounded to nearest even
                u32x2 pk[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    pk[tb].x = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{acc[tb][0], acc[tb][1]}, bf16x2));
                    pk[tb].y = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{acc[tb][2], acc[tb][3]}, bf16x2));
                }
                if constexpr (VEC) {
                    const BufRes wo = make_rsrc_window(ob16, T * z_row, t0 * z_row);
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb)
                        __builtin_amdgcn_raw_buffer_store_b64(
                            pk[tb], wo, off2 == kBufOOB ? kBufOOB : off2 + tb * 16 * static_cast<int>(z_row), 0, 0);
                } else {
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) {
                        const int64_t t = t0 + 16 * tb + c16;
                        const int col = v0 + 16 * wave + 4 * g4;
                        if (t < T) {
                            u16* dst = ob16 + (t * H + h) * static_cast<int64_t>(V) + col;
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (col + r < V) dst[r] = half_elem(pk[tb], r);
                        }
                    }
                }
            } else if constexpr (VEC) {
                const BufRes wo = make_rsrc_window(ob, T * o_row, t0 * o_row);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb)
                    buf_store16(__builtin_bit_cast(u32x4, acc[tb]), wo,
                                offo == kBufOOB ? kBufOOB : offo + tb * 16 * static_cast<int>(o_row));
            } else {
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    const int64_t t = t0 + 16 * tb + c16;
                    const int col = v0 + 16 * wave + 4 * g4;
                    if (t < T) {
                        float* dst = ob + t * H * static_cast<int64_t>(V) + h * static_cast<int64_t>(V) + col;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (col + r < V) dst[r] = acc[tb][r];
                    }
                }
            }
        }

        // state update: S = e^{G_L} o S + K~^T V~
        if constexpr (MODE == 0) {
            const float a = sDec[0];
#pragma unroll
            for (int db = 0; db < KB; ++db) S[db] *= a;
        } else {
            if (AGG || !fast) {
#pragma unroll
                for (int db = 0; db < KB; ++db) {
                    const f32x4 a = *reinterpret_cast<const f32x4*>(sEGL + 16 * db + 4 * g4);
                    S[db] *= a;
                }
            }
        }
        bf16x8 wBh[2], wBl[2];
        if constexpr (MODE == 0) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f32x4 w0 = *reinterpret_cast<const f32x4*>(sW + 32 * ks + 4 * g4);
                const f32x4 w1 = *reinterpret_cast<const f32x4*>(sW + 32 * ks + 16 + 4 * g4);
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(vA[ks][e]) * (e < 4 ? w0[e & 3] : w1[e & 3]);
                split8(x, wBh[ks], wBl[ks]);
            }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            // all key tiles' operands first, then the products term by term
            bf16x8 kh[KB];
#pragma unroll
            for (int db = 0; db < KB; ++db) kh[db] = tr_frag<LDK>(sK, 32 * ks, 16 * db, lane);
            if constexpr (MODE == 0) {
#pragma unroll
                for (int db = 0; db < KB; ++db) S[db] = mfma16(kh[db], wBl[ks], S[db]);
#pragma unroll
                for (int db = 0; db < KB; ++db) S[db] = mfma16(kh[db], wBh[ks], S[db]);
            } else {
                bf16x8 kl[KB];
#pragma unroll
                for (int db = 0; db < KB; ++db) kl[db] = tr_frag<LDK>(sK + L * LDK, 32 * ks, 16 * db, lane);
#pragma unroll
                for (int db = 0; db < KB; ++db) S[db] = mfma16(kl[db], vA[ks], S[db]);
#pragma unroll
                for (int db = 0; db < KB; ++db) S[db] = mfma16(kh[db], vA[ks], S[db]);
            }
        }
        __syncthreads();   // LDS operands are restaged by the next chunk
    }

    // ---- epilogue ----
    if constexpr (AGG) {
        float* ub = p.agg_u + ((static_cast<int64_t>(seg) * units + rest) * WPB + wave) * (KB * 256);
#pragma unroll
        for (int db = 0; db < KB; ++db) *reinterpret_cast<f32x4*>(ub + (db * 64 + lane) * 4) = S[db];
        if (vt == 0 && tid < KP) p.agg_a[(static_cast<int64_t>(seg) * p.B * H + bh) * KP + tid] = __expf(lsum);
    } else {
        if (seg == p.nseg - 1) {
#pragma unroll
            for (int db = 0; db < KB; ++db) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = 16 * db + 4 * g4 + r;
                    if (d < K && jcol < V)
                        p.s_final[((static_cast<int64_t>(b) * H + h) * K + d) * V + jcol] = S[db][r];
                }
            }
        }
    }
}

// Prefix over the segment states, in place, between the two passes: the
// segment pass leaves P_0 (segment 0 starts from s0) and, for s >= 1, the
// state U_s that segment s builds from zero with its decay product a_s; this
// makes P_s = a_s o P_{s-1} + U_s, the state after segment s, so each
// workgroup of the output pass loads one state.  One thread per (unit, wave,
// key tile, lane) owns 4 keys of one column; the loads of a batch of
// segments are issued before any of them is combined.
template <int KP, int WPB>
__global__ __launch_bounds__(256) void diag_segment_prefix_kernel(DiagArgs p) {
    constexpr int KB = KP / 16;
    constexpr int PER_UNIT = WPB * KB * 64;   // f32x4 per unit and segment
    constexpr int BATCH = 8;
    const int units = p.B * p.H * p.vtiles;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= static_cast<int64_t>(units) * PER_UNIT) return;
    const int unit = static_cast<int>(gid / PER_UNIT);
    const int rem = static_cast<int>(gid - static_cast<int64_t>(unit) * PER_UNIT);   // (wave, key tile, lane)
    const int db = (rem >> 6) % KB;
    const int g4 = (rem & 63) >> 4;
    const int bh = unit / p.vtiles;
    const int64_t ustride = static_cast<int64_t>(units) * PER_UNIT * 4;   // floats per segment
    const int64_t astride = static_cast<int64_t>(p.B) * p.H * KP;
    float* u = p.agg_u + (static_cast<int64_t>(unit) * PER_UNIT + rem) * 4;
    const float* a = p.agg_a + static_cast<int64_t>(bh) * KP + 16 * db + 4 * g4;
    f32x4 x = *reinterpret_cast<const f32x4*>(u);
    for (int s0 = 1; s0 < p.nseg - 1; s0 += BATCH) {
        f32x4 us[BATCH], as[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            if (s0 + j < p.nseg - 1) {
                us[j] = *reinterpret_cast<const f32x4*>(u + (s0 + j) * ustride);
                as[j] = *reinterpret_cast<const f32x4*>(a + (s0 + j) * astride);
            }
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            if (s0 + j < p.nseg - 1) {
                x = as[j] * x + us[j];
                *reinterpret_cast<f32x4*>(u + (s0 + j) * ustride) = x;
            }
        }
    }
}

template <int MODE, int KP, int WPB, bool KK>
hipError_t launch_t(const DiagArgs& a, bool vec, hipStream_t stream) {
    const int64_t units = static_cast<int64_t>(a.B) * a.H * a.vtiles;
    const dim3 block(64 * WPB);
    if (a.nseg > 1) {
        const dim3 grid(static_cast<unsigned>(units * (a.nseg - 1)));
        if (vec) hipLaunchKernelGGL((diag_outer_kernel<MODE, KP, WPB, true, true, KK>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((diag_outer_kernel<MODE, KP, WPB, false, true, KK>), grid, block, 0, stream, a);
        if (a.nseg > 2) {
            const int64_t threads = units * WPB * (KP / 16) * 64;
            hipLaunchKernelGGL((diag_segment_prefix_kernel<KP, WPB>), dim3(static_cast<unsigned>((threads + 255) / 256)),
                               dim3(256), 0, stream, a);
        }
    }
    const dim3 grid(static_cast<unsigned>(units * a.nseg));
    if (a.epi_kind != 0 || a.out_bf16) {
        if constexpr (!KK) {
            if (vec) hipLaunchKernelGGL((diag_outer_kernel<MODE, KP, WPB, true, false, false, true>), grid, block, 0,
                                        stream, a);
            else hipLaunchKernelGGL((diag_outer_kernel<MODE, KP, WPB, false, false, false, true>), grid, block, 0,
                                    stream, a);
            return hipGetLastError();
        } else {
            return hipErrorInvalidValue;   // the epilogue is not built for the per-key kappa variant
        }
    }
    if (vec) hipLaunchKernelGGL((diag_outer_kernel<MODE, KP, WPB, true, false, KK>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((diag_outer_kernel<MODE, KP, WPB, false, false, KK>), grid, block, 0, stream, a);
    return hipGetLastError();
}

// Output-pass workgroups that fit on one compute unit at once (LDS and
// registers), measured once per kernel variant.  Host threads driving separate
// contexts may ask at the same time: the cache is a relaxed atomic, and a
// race only repeats the (idempotent) query.
template <int MODE, int KP, int WPB, bool VEC, bool KK>
int resident_blocks() {
    static std::atomic<int> cached{0};
    int n = cached.load(std::memory_order_relaxed);
    if (n == 0) {
        int m = 1;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&m, diag_outer_kernel<MODE, KP, WPB, VEC, false, KK>,
                                                         64 * WPB, 0) != hipSuccess ||
            m < 1)
            m = 1;
        n = m;
        cached.store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int MODE, int KP, bool KK>
int resident_blocks_w(int wpb, bool vec) {
    if (wpb == 8) return vec ? resident_blocks<MODE, KP, 8, true, KK>() : resident_blocks<MODE, KP, 8, false, KK>();
    return vec ? resident_blocks<MODE, KP, 4, true, KK>() : resident_blocks<MODE, KP, 4, false, KK>();
}

int resident_blocks(int decay_mode, bool kk, int K, int wpb, bool vec) {
    if (decay_mode == 0)
        return K <= 64 ? resident_blocks_w<0, 64, false>(wpb, vec) : resident_blocks_w<0, 128, false>(wpb, vec);
    if (kk) return K <= 64 ? resident_blocks_w<1, 64, true>(wpb, vec) : resident_blocks_w<1, 128, true>(wpb, vec);
    return K <= 64 ? resident_blocks_w<1, 64, false>(wpb, vec) : resident_blocks_w<1, 128, false>(wpb, vec);
}

template <int MODE, int KP, bool KK>
hipError_t launch_w(const DiagArgs& a, int wpb, bool vec, hipStream_t stream) {
    return wpb == 8 ? launch_t<MODE, KP, 8, KK>(a, vec, stream) : launch_t<MODE, KP, 4, KK>(a, vec, stream);
}

}  // namespace

DiagPlan diag_outer_plan(int B, int T, int H, int V, int K, int decay_mode, bool kscale_key, bool vec,
                         int num_cus, int requested_segments) {
    DiagPlan pl{};
    pl.waves = waves_for(V);
    const int vt = 16 * pl.waves;
    pl.nchunks = (T + L - 1) / L;
    pl.vtiles = (V + vt - 1) / vt;
    const int64_t units = static_cast<int64_t>(B) * H * pl.vtiles;
    int64_t nseg = requested_segments;
    if (nseg <= 0) {
        // Segments to fill the chip's resident workgroup slots: once where a
        // compute unit holds one workgroup (wide per-key heads), twice where it
        // holds two or more (the second round covers the tail of the first);
        // at least kMinChunksPerSegment chunks each, since every extra
        // segment adds a reduction pass over its chunks.  Measured on the
        // Mamba-2, GLA, HGRN2 and associative-memory shapes.  Where a compute
        // unit holds one workgroup (8-wave per-key variants), filling the chip
        // outweighs the extra reduction on short or narrow calls: segments
        // down to 2 chunks (GLA B=4 T=1024 54.7 -> 38.6 us, B=1 T=4096
        // 56.0 -> 41.1 us; the benchmark shapes keep their counts).
        const int res = resident_blocks(decay_mode, kscale_key, K, pl.waves, vec);
        const int64_t slots = static_cast<int64_t>(num_cus) * res;
        nseg = (res >= 2 ? 2 * slots : slots) / units;
        const int minc = res >= 2 ? kMinChunksPerSegment : 2;
        if (nseg > pl.nchunks / minc) nseg = pl.nchunks / minc;
    }
    if (nseg > pl.nchunks) nseg = pl.nchunks;
    if (nseg < 1) nseg = 1;
    pl.cps = static_cast<int>((pl.nchunks + nseg - 1) / nseg);
    pl.nseg = (pl.nchunks + pl.cps - 1) / pl.cps;
    return pl;
}

size_t diag_outer_workspace_bytes(int B, int H, int K, int V, int nseg) {
    if (nseg <= 1) return 0;
    const size_t kp = K <= 64 ? 64 : 128, vt = 16 * static_cast<size_t>(waves_for(V));
    const size_t vtiles = (static_cast<size_t>(V) + vt - 1) / vt;
    return static_cast<size_t>(nseg - 1) * B * H * (vtiles * kp * vt + kp) * sizeof(float);
}

hipError_t launch_scan_diag_outer(const DiagParams& prm, const DiagPlan& pl, void* workspace, hipStream_t stream) {
    DiagArgs a{};
    a.q = reinterpret_cast<const u16*>(prm.q);
    a.k = reinterpret_cast<const u16*>(prm.k);
    a.v = reinterpret_cast<const u16*>(prm.v);
    a.g = prm.g;
    a.ks = prm.k_scale;
    a.s0 = prm.s0;
    a.o = prm.o;
    a.s_final = prm.s_final;
    a.B = prm.B;
    a.T = prm.T;
    a.H = prm.H;
    a.Hg = prm.Hg;
    a.K = prm.K;
    a.V = prm.V;
    a.scale = prm.scale;
    a.vtiles = pl.vtiles;
    a.nchunks = pl.nchunks;
    a.nseg = pl.nseg;
    a.cps = pl.cps;
    a.epi_kind = prm.epi_kind;
    a.out_bf16 = prm.out_bf16;
    a.d_skip = prm.d_skip;
    a.gate = reinterpret_cast<const u16*>(prm.gate);
    a.norm_w = prm.norm_w;
    a.eps = prm.eps;
    if (pl.nseg > 1) {
        const size_t kp = prm.K <= 64 ? 64 : 128;
        a.agg_u = static_cast<float*>(workspace);
        a.agg_a = a.agg_u + static_cast<size_t>(pl.nseg - 1) * prm.B * prm.H * pl.vtiles * kp * (16 * pl.waves);
    }
    const bool vec = prm.vec != 0;
    const bool k64 = prm.K <= 64;
    if (prm.decay_mode == 0)
        return k64 ? launch_w<0, 64, false>(a, pl.waves, vec, stream) : launch_w<0, 128, false>(a, pl.waves, vec, stream);
    if (prm.k_scale_key)
        return k64 ? launch_w<1, 64, true>(a, pl.waves, vec, stream) : launch_w<1, 128, true>(a, pl.waves, vec, stream);
    return k64 ? launch_w<1, 64, false>(a, pl.waves, vec, stream) : launch_w<1, 128, false>(a, pl.waves, vec, stream);
}

}  // namespace lrs
