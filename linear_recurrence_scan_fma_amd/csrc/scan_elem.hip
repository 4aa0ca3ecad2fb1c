// Elementwise first-order scans on gfx950:
//   FMA form    s_t = a_t s_{t-1} + b_t
//   gated form  s_t = a_t s_{t-1} + (1 - a_t) u_t   (evaluated as fma(a, s, (1 - a) u))
// [SunnyNet log §2.1: "SunnyNet 工程化实录：一个 O(N) 架构如何长出自己的 C 推理运行时",
//  developer.aliyun.com/article/1773847 -- the unified kernel's two forms].
//
// Both forms are affine maps s -> A s + B, and composing two steps gives
// (A2 A1, A2 B1 + B2).  The scan is computed on (A, B) pairs:
//
//  * Layout: [B,T,N] fp32, channels contiguous.  A workgroup (4 waves) owns a
//    tile of NC = 16*VEC channels.  Inside a wave, 16 lanes run along the
//    channels (VEC channels each, one float4 per lane per row when VEC = 4)
//    and 4 lanes along time; the 4 waves stack further along time.  So a
//    chunk is 16 time-lanes x R rows, and each lane owns R consecutive rows.
//  * Per chunk: every lane folds its R rows into one (A, B) pair per channel,
//    the 4 time-lanes of a wave combine by cross-lane shuffles (an inclusive
//    Hillis-Steele scan over lanes 16 apart), the 4 waves combine through LDS,
//    and each lane then replays its rows from its exact carry-in and streams
//    the states out.  Inputs are held in registers between the load and the
//    replay, so every input byte crosses HBM once and every output byte once.
//  * Across chunks, two schedules:
//      stream:   a workgroup walks the whole time axis of its channel tile,
//                prefetching chunk c+1 while it scans chunk c; the carry stays
//                in registers.  No inter-workgroup traffic at all.
//      lookback: a workgroup owns a single chunk of a channel tile (the
//                default whenever there are several chunks).  It
//                publishes its chunk aggregate, then walks back over
//                predecessors' status words until it finds an inclusive
//                prefix (decoupled look-back), then publishes its own
//                inclusive prefix.  Used when there are too few channel tiles
//                to fill the GPU.  Status words pack (epoch, fp32 value) into
//                one 64-bit word written and read with agent-scope atomics,
//                so a word is valid exactly when its tag equals this call's
//                epoch: no fences, no reset between calls.  Tiles are taken
//                in order from an atomic counter, so every predecessor of a
//                running tile has already been taken by a running or finished
//                workgroup, and aggregates never wait on anything: the walk
//                always terminates.  It is additionally bounded in wall time.
#include <mutex>

#include "lrs_internal.h"

namespace lrs {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChanLanes = 16;                     // lanes along channels per wave
constexpr int kTimeLanesPerWave = 64 / kChanLanes; // 4
constexpr int kTimeLanes = kWaves * kTimeLanesPerWave;  // 16
constexpr unsigned long long kSpinTicks = 1ull << 29;   // ~5 s of the 100 MHz real-time counter

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct ElemArgs {
    const float* a;
    const float* x;
    const float* s0;
    float* s;
    float* s_final;
    int64_t T, N;
    int64_t chan_tiles;   // channel tiles per batch row
    int64_t ncols;        // B * chan_tiles
    int64_t nchunks;
    unsigned long long* words;
    unsigned long long* counter;
    unsigned long long counter_base;
    unsigned int epoch;
    unsigned int* error_flag;
    unsigned int delay_seed;   // scrambled-arrival variant only: seeds its delays
};

// Scrambled-arrival variant of the look-back (a verification tool): before a
// tile publishes its aggregate, before it walks back and before it publishes
// its inclusive prefix, its look-back wave sleeps a pseudo-random time (0 to
// about 4 us, from a hash of the seed, the tile and the point), so tiles
// arrive at the status words in an order unrelated to the normal timing.
__device__ __forceinline__ void scramble_delay(unsigned int seed, int64_t tile, unsigned int point) {
    unsigned int x = seed ^ (static_cast<unsigned int>(tile) * 0x9e3779b9u) ^ (point * 0x85ebca6bu);
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    const unsigned int n = x & 63u;   // 0 .. 63 sleeps of 64 x 2 cycles
    for (unsigned int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(2);
}

// One step of either update.  The gated form is evaluated as written,
// a s + (1 - a) u [SunnyNet log §2.1], with 1 - a exact for a in [0.5, 1]:
// the rounding of the injected term then scales with 1 - a.  (The
// rearranged a (s - u) + u rounds s - u at the size of u and keeps that
// error whole; with gates near 1, whose errors persist for ~1 / (1 - a)
// steps, it measured 4.8e-5 normwise against 6.5e-7 for this form, for
// a = 1 - U(0, 1e-3) over 65,613 steps.)  The state's dependence chain is one
// fma either way.
template <bool GATED>
__device__ __forceinline__ float step(float a, float x, float s) {
    if constexpr (GATED) {
        return __builtin_fmaf(a, s, (1.0f - a) * x);
    } else {
        return __builtin_fmaf(a, s, x);
    }
}

template <int VEC>
__device__ __forceinline__ void load_vec(const float* p, float (&v)[VEC]) {
    if constexpr (VEC == 4) {
        f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else {
        v[0] = __builtin_nontemporal_load(p);
    }
}

template <int VEC>
__device__ __forceinline__ void store_vec(float* p, const float (&v)[VEC]) {
    if constexpr (VEC == 4) {
        f32x4 t = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(p));
    } else {
        __builtin_nontemporal_store(v[0], p);
    }
}

__device__ __forceinline__ unsigned long long pack_word(unsigned int epoch, float v) {
    return (static_cast<unsigned long long>(epoch) << 32) | __float_as_uint(v);
}

__device__ __forceinline__ void publish(unsigned long long* w, unsigned int epoch, float v) {
    __hip_atomic_store(w, pack_word(epoch, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long poll(const unsigned long long* w) {
    return __hip_atomic_load(const_cast<unsigned long long*>(w), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// Walks back from tile `pred` (same channel column, earlier chunk) composing
// aggregates until an inclusive prefix is found; returns the carry-in.
__device__ float look_back(const ElemArgs& p, int64_t pred, int c, int nc) {
    float accA = 1.0f, accB = 0.0f;  // maps of the tiles between pred and the caller
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    while (true) {
        const unsigned long long wi = poll(p.words + (pred * 3 + 2) * nc + c);
        if (static_cast<unsigned int>(wi >> 32) == p.epoch) {
            return __builtin_fmaf(accA, __uint_as_float(static_cast<unsigned int>(wi)), accB);
        }
        if (pred >= p.ncols) {  // chunk 0 tiles publish only inclusive prefixes
            const unsigned long long wa = poll(p.words + (pred * 3 + 0) * nc + c);
            const unsigned long long wb = poll(p.words + (pred * 3 + 1) * nc + c);
            if (static_cast<unsigned int>(wa >> 32) == p.epoch &&
                static_cast<unsigned int>(wb >> 32) == p.epoch) {
                const float pa = __uint_as_float(static_cast<unsigned int>(wa));
                const float pb = __uint_as_float(static_cast<unsigned int>(wb));
                accB = __builtin_fmaf(accA, pb, accB);  // pred's map first, then acc
                accA = accA * pa;
                pred -= p.ncols;
                continue;
            }
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
            __hip_atomic_store(p.error_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return __builtin_nanf("");
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// The channel column and chunk range this workgroup scans.  Stream: column
// blockIdx.x, every chunk.  Look-back: the next tile from the counter (tiles
// are numbered chunk-major), one chunk.  Returns false, after flagging the
// error, when the counter is out of step with this launch.
template <bool LOOKBACK>
__device__ __forceinline__ bool take_tile(const ElemArgs& p, int tid, long long& sh_tile, int64_t& col,
                                          int64_t& chunk_lo, int64_t& chunk_hi, int64_t& tile) {
    tile = 0;
    if constexpr (LOOKBACK) {
        if (tid == 0) {
            sh_tile = static_cast<long long>(
                __hip_atomic_fetch_add(p.counter, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                p.counter_base);
        }
        __syncthreads();
        tile = sh_tile;
        if (tile < 0 || tile >= p.ncols * p.nchunks) {
            if (tid == 0)
                __hip_atomic_store(p.error_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        chunk_lo = tile / p.ncols;
        chunk_hi = chunk_lo + 1;
        col = tile - chunk_lo * p.ncols;
    } else {
        col = blockIdx.x;
        chunk_lo = 0;
        chunk_hi = p.nchunks;
    }
    return true;
}

// Phases 2-4 of one chunk, shared by the forward and reverse kernels.  On
// entry (A, Bv) is the affine map of this lane's rows, folded in order; on
// exit `st` is the state entering this lane's first row.  The stream schedule
// keeps the state entering the chunk in `carry` and advances it past the
// chunk here; the look-back schedule fetches it through the status words,
// starting from p.s0 at chunk 0.  One barrier per chunk (two with look-back):
// `tot` alternates between two buffers on consecutive chunks.
template <int VEC, bool LOOKBACK, bool SCR>
__device__ __forceinline__ void lane_carry_in(const ElemArgs& p, int64_t chunk, int64_t tile, int64_t b,
                                              int64_t jt, int lane, int wave, int cl, int tlw,
                                              float (&A)[VEC], float (&Bv)[VEC], float (&carry)[VEC],
                                              float (&st)[VEC], float (&tot)[kWaves][2][kChanLanes * VEC],
                                              float (&sh_carry)[kChanLanes * VEC]) {
    constexpr int NC = kChanLanes * VEC;
    // inclusive scan over the 4 time-lanes of the wave (lanes 16 apart)
#pragma unroll
    for (int off = kChanLanes; off < 64; off <<= 1) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const float pA = __shfl_up(A[v], off);
            const float pB = __shfl_up(Bv[v], off);
            if (lane >= off) {
                Bv[v] = __builtin_fmaf(A[v], pB, Bv[v]);
                A[v] = A[v] * pA;
            }
        }
    }
    // exclusive prefix inside the wave
    float eA[VEC], eB[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        const float pA = __shfl_up(A[v], kChanLanes);
        const float pB = __shfl_up(Bv[v], kChanLanes);
        eA[v] = tlw == 0 ? 1.0f : pA;
        eB[v] = tlw == 0 ? 0.0f : pB;
    }
    // wave totals through LDS
    if (tlw == kTimeLanesPerWave - 1) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            tot[wave][0][cl * VEC + v] = A[v];
            tot[wave][1][cl * VEC + v] = Bv[v];
        }
    }
    __syncthreads();

    if constexpr (LOOKBACK) {
        if (wave == 0 && lane < NC) {
            const int c = lane;
            float TA = 1.0f, TB = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float wa = tot[w][0][c];
                const float wb = tot[w][1][c];
                TB = __builtin_fmaf(wa, TB, wb);
                TA = TA * wa;
            }
            float cin;
            if (chunk == 0) {
                const int64_t ch = jt * NC + c;
                cin = (p.s0 && ch < p.N) ? p.s0[b * p.N + ch] : 0.0f;
            } else {
                if constexpr (SCR) scramble_delay(p.delay_seed, tile, 0u);
                publish(p.words + (tile * 3 + 0) * NC + c, p.epoch, TA);
                publish(p.words + (tile * 3 + 1) * NC + c, p.epoch, TB);
                if constexpr (SCR) scramble_delay(p.delay_seed, tile, 1u);
                cin = look_back(p, tile - p.ncols, c, NC);
            }
            if constexpr (SCR) scramble_delay(p.delay_seed, tile, 2u);
            publish(p.words + (tile * 3 + 2) * NC + c, p.epoch, __builtin_fmaf(TA, cin, TB));
            sh_carry[c] = cin;
        }
        __syncthreads();
#pragma unroll
        for (int v = 0; v < VEC; ++v) carry[v] = sh_carry[cl * VEC + v];
    }

    // this lane's carry-in: waves before it, then lanes before it in its wave
    float PA[VEC], PB[VEC], TA[VEC], TB[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) { PA[v] = 1.0f; PB[v] = 0.0f; TA[v] = 1.0f; TB[v] = 0.0f; }
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const float wa = tot[w][0][cl * VEC + v];
            const float wb = tot[w][1][cl * VEC + v];
            if (w < wave) {
                PB[v] = __builtin_fmaf(wa, PB[v], wb);
                PA[v] = PA[v] * wa;
            }
            TB[v] = __builtin_fmaf(wa, TB[v], wb);
            TA[v] = TA[v] * wa;
        }
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        const float xa = eA[v] * PA[v];
        const float xb = __builtin_fmaf(eA[v], PB[v], eB[v]);
        st[v] = __builtin_fmaf(xa, carry[v], xb);
        carry[v] = __builtin_fmaf(TA[v], carry[v], TB[v]);   // stream schedule: past this chunk
    }
}

template <bool GATED, int VEC, int R, bool LOOKBACK, bool SCR = false>
__global__ __launch_bounds__(kThreads) void scan_elem_kernel(ElemArgs p) {
    constexpr int NC = kChanLanes * VEC;   // channels per tile
    constexpr int CH = kTimeLanes * R;     // rows per chunk

    __shared__ float sh_tot[2][kWaves][2][NC];
    __shared__ float sh_carry[NC];
    __shared__ long long sh_tile;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cl = lane & (kChanLanes - 1);
    const int tlw = lane / kChanLanes;
    const int tl = wave * kTimeLanesPerWave + tlw;

    int64_t col, chunk_lo, chunk_hi, tile;
    if (!take_tile<LOOKBACK>(p, tid, sh_tile, col, chunk_lo, chunk_hi, tile)) return;
    const int64_t b = col / p.chan_tiles;
    const int64_t jt = col - b * p.chan_tiles;
    const int64_t ch0 = jt * NC + cl * VEC;
    const bool chan_ok = ch0 < p.N;   // VEC = 4 only when N % 4 == 0
    const int64_t base = b * p.T * p.N + ch0;

    float carry[VEC];
    if constexpr (!LOOKBACK) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) carry[v] = (p.s0 && chan_ok) ? p.s0[b * p.N + ch0 + v] : 0.0f;
    }

    float ca[R][VEC], cx[R][VEC];
    auto load_chunk = [&](int64_t chunk, float (&A)[R][VEC], float (&X)[R][VEC]) {
        const int64_t row0 = chunk * CH + static_cast<int64_t>(tl) * R;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = row0 + r;
            if (chan_ok && row < p.T) {
                load_vec<VEC>(p.a + base + row * p.N, A[r]);
                load_vec<VEC>(p.x + base + row * p.N, X[r]);
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v) { A[r][v] = 1.0f; X[r][v] = 0.0f; }
            }
        }
    };
    load_chunk(chunk_lo, ca, cx);

    for (int64_t chunk = chunk_lo; chunk < chunk_hi; ++chunk) {
        float na[R][VEC], nx[R][VEC];
        const bool has_next = !LOOKBACK && chunk + 1 < chunk_hi;   // look-back tiles are one chunk
        if (has_next) load_chunk(chunk + 1, na, nx);

        const int64_t row0 = chunk * CH + static_cast<int64_t>(tl) * R;
        const int64_t rem = chan_ok ? p.T - row0 : 0;   // lanes past N store nothing
        const int nvalid = rem <= 0 ? 0 : (rem >= R ? R : static_cast<int>(rem));

        // 1. fold this lane's rows into one affine pair per channel
        float A[VEC], Bv[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) { A[v] = 1.0f; Bv[v] = 0.0f; }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r < nvalid) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    A[v] *= ca[r][v];
                    Bv[v] = step<GATED>(ca[r][v], cx[r][v], Bv[v]);
                }
            }
        }
        float st[VEC];
        lane_carry_in<VEC, LOOKBACK, SCR>(p, chunk, tile, b, jt, lane, wave, cl, tlw, A, Bv, carry, st,
                                     sh_tot[chunk & 1], sh_carry);

        // 5. replay this lane's rows from the exact carry-in and stream states out
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r < nvalid) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) st[v] = step<GATED>(ca[r][v], cx[r][v], st[v]);
                const int64_t row = row0 + r;
                store_vec<VEC>(p.s + base + row * p.N, st);
                if (row == p.T - 1) {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) p.s_final[b * p.N + ch0 + v] = st[v];
                }
            }
        }
        if (has_next) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int v = 0; v < VEC; ++v) { ca[r][v] = na[r][v]; cx[r][v] = nx[r][v]; }
        }
    }
}

// Reverse (gradient) pass.  With gs_t the loss gradient reaching state s_t,
//   gs_T = ds_T + ds_final,   gs_t = ds_t + a_{t+1} gs_{t+1},
// which is the FMA scan G_j = alpha_j G_{j-1} + beta_j run over reversed
// steps j = T-1-t (0-based rows): alpha_j = a at row t+1 (1 for the last
// row), beta_j = ds at row t, G_{-1} = ds_final.  The chunk, look-back and
// carry machinery is the forward kernel's, unchanged; only the rows a lane
// reads differ.  Each gs_t is consumed where it is produced:
//   FMA form    da_t = gs_t s_{t-1}            db_t = gs_t
//   gated form  da_t = gs_t (s_{t-1} - u_t)     du_t = gs_t (1 - a_t)
//   ds0 = a_1 gs_1 (row 0), with s_{t-1} the forward state of the row before
// (s0 for row 0).  So the pass reads a, ds, s (and u) once and writes da and
// db (or du) once: 20 bytes per element for the FMA form, 24 for the gated.
struct ElemBwdArgs {
    ElemArgs sc;          // the reverse scan's shape, look-back state and initial value (ds_final)
    const float* a;       // forward coefficients [B,T,N]
    const float* u;       // gated inputs [B,T,N] (gated form only)
    const float* s0;      // forward initial state [B,N], nullable
    const float* s;       // forward states [B,T,N]
    const float* ds;      // incoming gradients [B,T,N]
    float* da;
    float* dx;            // db or du
    float* ds0;           // [B,N], nullable
};

template <bool GATED, int VEC, int R, bool LOOKBACK, bool SCR = false>
__global__ __launch_bounds__(kThreads) void scan_elem_bwd_kernel(ElemBwdArgs q) {
    constexpr int NC = kChanLanes * VEC;
    constexpr int CH = kTimeLanes * R;
    // a lane's reversed rows j0 .. j0+R-1 are forward rows T-1-j0 down to
    // T-j0-R; it reads a at forward rows T-j0 down to T-j0-R+1 as alpha, and
    // the gated form also needs a at the lane's own rows: one row more
    constexpr int NA = GATED ? R + 1 : R;
    const ElemArgs& p = q.sc;

    __shared__ float sh_tot[2][kWaves][2][NC];
    __shared__ float sh_carry[NC];
    __shared__ long long sh_tile;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int cl = lane & (kChanLanes - 1);
    const int tlw = lane / kChanLanes;
    const int tl = wave * kTimeLanesPerWave + tlw;

    int64_t col, chunk_lo, chunk_hi, tile;
    if (!take_tile<LOOKBACK>(p, tid, sh_tile, col, chunk_lo, chunk_hi, tile)) return;
    const int64_t b = col / p.chan_tiles;
    const int64_t jt = col - b * p.chan_tiles;
    const int64_t ch0 = jt * NC + cl * VEC;
    const bool chan_ok = ch0 < p.N;
    const int64_t base = b * p.T * p.N + ch0;
    const int64_t T = p.T;

    float carry[VEC];
    if constexpr (!LOOKBACK) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) carry[v] = (p.s0 && chan_ok) ? p.s0[b * p.N + ch0 + v] : 0.0f;
    }

    // ca[r] = a at forward row T - j0 - r (1 outside [0, T)), cd[r] = ds at
    // forward row T-1-j0-r (0 outside)
    float ca[NA][VEC], cd[R][VEC];
    auto load_chunk = [&](int64_t chunk, float (&A)[NA][VEC], float (&D)[R][VEC]) {
        const int64_t j0 = chunk * CH + static_cast<int64_t>(tl) * R;
#pragma unroll
        for (int r = 0; r < NA; ++r) {
            const int64_t row = T - j0 - r;
            if (chan_ok && row >= 0 && row < T) {
                load_vec<VEC>(q.a + base + row * p.N, A[r]);
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v) A[r][v] = 1.0f;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = T - 1 - j0 - r;
            if (chan_ok && row >= 0) {
                load_vec<VEC>(q.ds + base + row * p.N, D[r]);
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v) D[r][v] = 0.0f;
            }
        }
    };
    load_chunk(chunk_lo, ca, cd);

    for (int64_t chunk = chunk_lo; chunk < chunk_hi; ++chunk) {
        const int64_t j0 = chunk * CH + static_cast<int64_t>(tl) * R;
        const int64_t rem = chan_ok ? T - j0 : 0;
        const int nvalid = rem <= 0 ? 0 : (rem >= R ? R : static_cast<int>(rem));

        // the epilogue's operands: s at the row before each of the lane's rows
        // (s0 before row 0), and u at the rows themselves
        float sp[R][VEC], cu[R][VEC];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = T - 1 - j0 - r;
            if (chan_ok && row >= 1) {
                load_vec<VEC>(q.s + base + (row - 1) * p.N, sp[r]);
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    sp[r][v] = (row == 0 && q.s0 && chan_ok) ? q.s0[b * p.N + ch0 + v] : 0.0f;
            }
            if constexpr (GATED) {
                if (chan_ok && row >= 0) {
                    load_vec<VEC>(q.u + base + row * p.N, cu[r]);
                } else {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) cu[r][v] = 0.0f;
                }
            }
        }

        float na[NA][VEC], nd[R][VEC];
        const bool has_next = !LOOKBACK && chunk + 1 < chunk_hi;   // look-back tiles are one chunk
        if (has_next) load_chunk(chunk + 1, na, nd);

        // fold this lane's reversed rows: G -> alpha G + beta
        float A[VEC], Bv[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) { A[v] = 1.0f; Bv[v] = 0.0f; }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r < nvalid) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    A[v] *= ca[r][v];
                    Bv[v] = __builtin_fmaf(ca[r][v], Bv[v], cd[r][v]);
                }
            }
        }
        float g[VEC];
        lane_carry_in<VEC, LOOKBACK, SCR>(p, chunk, tile, b, jt, lane, wave, cl, tlw, A, Bv, carry, g,
                                     sh_tot[chunk & 1], sh_carry);

        // replay from the exact carry-in; gradients of this lane's rows
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r < nvalid) {
                const int64_t row = T - 1 - j0 - r;
                float da[VEC], dx[VEC];
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    g[v] = __builtin_fmaf(ca[r][v], g[v], cd[r][v]);
                    if constexpr (GATED) {
                        da[v] = g[v] * (sp[r][v] - cu[r][v]);
                        dx[v] = g[v] * (1.0f - ca[r + 1][v]);
                    } else {
                        da[v] = g[v] * sp[r][v];
                        dx[v] = g[v];
                    }
                }
                store_vec<VEC>(q.da + base + row * p.N, da);
                store_vec<VEC>(q.dx + base + row * p.N, dx);
                if (row == 0 && q.ds0) {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) q.ds0[b * p.N + ch0 + v] = q.a[base + v] * g[v];
                }
            }
        }
        if (has_next) {
#pragma unroll
            for (int r = 0; r < NA; ++r)
#pragma unroll
                for (int v = 0; v < VEC; ++v) ca[r][v] = na[r][v];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int v = 0; v < VEC; ++v) cd[r][v] = nd[r][v];
        }
    }
}

// One in-place time step for n channels, s = step(a, x, s): a pure stream of
// 16 bytes per channel (three reads, one write), one float4 per lane.
// Streaming (non-temporal) accesses measured faster than cached ones at every
// size from 0.8 M channels up, and no slower below.
template <bool GATED, bool VEC4>
__global__ __launch_bounds__(kThreads) void step_elem_kernel(const float* a, const float* x, float* s,
                                                              int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if constexpr (VEC4) {
        const int64_t n4 = n / 4;
        for (; i < n4; i += stride) {
            const f32x4 va = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a) + i);
            const f32x4 vx = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x) + i);
            f32x4 vs = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(s) + i);
            vs.x = step<GATED>(va.x, vx.x, vs.x);
            vs.y = step<GATED>(va.y, vx.y, vs.y);
            vs.z = step<GATED>(va.z, vx.z, vs.z);
            vs.w = step<GATED>(va.w, vx.w, vs.w);
            __builtin_nontemporal_store(vs, reinterpret_cast<f32x4*>(s) + i);
        }
    } else {
        for (; i < n; i += stride)
            __builtin_nontemporal_store(step<GATED>(__builtin_nontemporal_load(a + i), __builtin_nontemporal_load(x + i),
                                                    __builtin_nontemporal_load(s + i)),
                                        s + i);
    }
}

__global__ void fill_zero_u64_kernel(unsigned long long* p, size_t n) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        p[i] = 0ull;
}

template <bool GATED, int VEC, int R>
hipError_t launch_variant(const ElemArgs& a, bool lookback, int64_t grid, hipStream_t stream) {
    if (lookback && a.delay_seed) {
        hipLaunchKernelGGL((scan_elem_kernel<GATED, VEC, R, true, true>), dim3(static_cast<unsigned>(grid)),
                           dim3(kThreads), 0, stream, a);
    } else if (lookback) {
        hipLaunchKernelGGL((scan_elem_kernel<GATED, VEC, R, true>), dim3(static_cast<unsigned>(grid)),
                           dim3(kThreads), 0, stream, a);
    } else {
        hipLaunchKernelGGL((scan_elem_kernel<GATED, VEC, R, false>), dim3(static_cast<unsigned>(grid)),
                           dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

template <bool GATED, int VEC>
hipError_t launch_rows(const ElemArgs& a, const ElemPlan& plan, bool lookback, hipStream_t s) {
    switch (plan.rows) {
        case 2: return launch_variant<GATED, VEC, 2>(a, lookback, plan.grid, s);
        case 4: return launch_variant<GATED, VEC, 4>(a, lookback, plan.grid, s);
        case 16: return launch_variant<GATED, VEC, 16>(a, lookback, plan.grid, s);
        default: return launch_variant<GATED, VEC, 8>(a, lookback, plan.grid, s);
    }
}

template <bool GATED>
hipError_t launch_gated(const ElemArgs& a, const ElemPlan& plan, bool lookback, hipStream_t s) {
    return plan.vec == 4 ? launch_rows<GATED, 4>(a, plan, lookback, s) : launch_rows<GATED, 1>(a, plan, lookback, s);
}

template <bool GATED, int VEC, int R>
hipError_t launch_bwd_variant(const ElemBwdArgs& a, bool lookback, int64_t grid, hipStream_t stream) {
    if (lookback && a.sc.delay_seed) {
        hipLaunchKernelGGL((scan_elem_bwd_kernel<GATED, VEC, R, true, true>), dim3(static_cast<unsigned>(grid)),
                           dim3(kThreads), 0, stream, a);
    } else if (lookback) {
        hipLaunchKernelGGL((scan_elem_bwd_kernel<GATED, VEC, R, true>), dim3(static_cast<unsigned>(grid)),
                           dim3(kThreads), 0, stream, a);
    } else {
        hipLaunchKernelGGL((scan_elem_bwd_kernel<GATED, VEC, R, false>), dim3(static_cast<unsigned>(grid)),
                           dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

template <bool GATED, int VEC>
hipError_t launch_bwd_rows(const ElemBwdArgs& a, const ElemPlan& plan, bool lookback, hipStream_t s) {
    switch (plan.rows) {
        case 2: return launch_bwd_variant<GATED, VEC, 2>(a, lookback, plan.grid, s);
        case 8: return launch_bwd_variant<GATED, VEC, 8>(a, lookback, plan.grid, s);
        default: return hipErrorInvalidValue;
    }
}

template <bool GATED>
hipError_t launch_bwd_gated(const ElemBwdArgs& a, const ElemPlan& plan, bool lookback, hipStream_t s) {
    return plan.vec == 4 ? launch_bwd_rows<GATED, 4>(a, plan, lookback, s)
                         : launch_bwd_rows<GATED, 1>(a, plan, lookback, s);
}

ElemArgs scan_args(const ElemParams& p, const ElemPlan& plan) {
    ElemArgs a{};
    a.a = p.a;
    a.x = p.x;
    a.s0 = p.s0;
    a.s = p.s;
    a.s_final = p.s_final;
    a.T = p.T;
    a.N = p.N;
    a.chan_tiles = plan.chan_tiles;
    a.ncols = p.B * plan.chan_tiles;
    a.nchunks = plan.chunks;
    a.words = p.words;
    a.counter = p.counter;
    a.counter_base = p.counter_base;
    a.epoch = p.epoch;
    a.error_flag = p.error_flag;
    a.delay_seed = p.delay_seed;
    return a;
}

}  // namespace

ElemPlan elem_plan(int64_t B, int64_t T, int64_t N, bool aligned16, int schedule) {
    ElemPlan pl{};
    pl.vec = (aligned16 && N % 4 == 0) ? 4 : 1;
    const int64_t nc = kChanLanes * pl.vec;
    pl.chan_tiles = (N + nc - 1) / nc;
    if (schedule == kElemStream) {
        pl.rows = 8;
    } else {
        // short sequences get short chunks so that the look-back has tiles to chain
        pl.rows = T >= 4 * kTimeLanes * 8 ? 8 : 2;
    }
    const int64_t ch = kTimeLanes * pl.rows;
    pl.chunks = (T + ch - 1) / ch;
    if (schedule == kElemStream) {
        pl.grid = B * pl.chan_tiles;
        pl.words = 0;
    } else {
        pl.grid = B * pl.chan_tiles * pl.chunks;
        pl.words = static_cast<size_t>(pl.grid) * 3 * static_cast<size_t>(nc);
    }
    return pl;
}

// The look-back schedule takes tiles in time-major order, so at any moment the
// running workgroups cover a compact band of rows of every tensor; measured on
// the B=16 T=8192 N=2048 gated workload it streams at 5.8 TB/s against 4.9 TB/s
// for the stream schedule (whose workgroups each sweep their own column strip
// over the whole time axis).  Where the look-back grid is larger than the
// resident workgroup slots, its chunk-major tiles run in rounds, and each round
// pays a load, publish and poll latency (~7 us per chunk row at B=16 N=2048);
// so the stream schedule is taken when its own walk is a single chunk, or when
// it has a workgroup for every compute unit and at most 8 chunks to walk
// (T <= 1024: B=16 T=128 N=2048 6.8 against 31.6 us, T=1024 77 against 84 us;
// at T=2048 the two tie, and from T=4096 on the look-back wins).  Otherwise
// the look-back, while there are two or more chunks and its status words stay
// within 256 MB.
int elem_auto_schedule(int64_t B, int64_t T, int64_t N, bool aligned16, int num_cus) {
    const ElemPlan lb = elem_plan(B, T, N, aligned16, kElemLookback);
    if (lb.chunks <= 1 || lb.words * sizeof(unsigned long long) > (size_t{256} << 20)) return kElemStream;
    const ElemPlan st = elem_plan(B, T, N, aligned16, kElemStream);
    if (st.chunks <= 1 || (st.grid >= num_cus && st.chunks <= 8)) return kElemStream;
    return kElemLookback;
}

hipError_t launch_scan_elem(const ElemParams& p, const ElemPlan& plan, hipStream_t stream) {
    const ElemArgs a = scan_args(p, plan);
    const bool lookback = p.schedule == kElemLookback;
    return p.gated ? launch_gated<true>(a, plan, lookback, stream)
                   : launch_gated<false>(a, plan, lookback, stream);
}

hipError_t launch_scan_elem_bwd(const ElemBwdParams& p, const ElemPlan& plan, hipStream_t stream) {
    ElemBwdArgs a{};
    a.sc = scan_args(p.scan, plan);
    a.a = p.a;
    a.u = p.u;
    a.s0 = p.s0;
    a.s = p.s;
    a.ds = p.ds;
    a.da = p.da;
    a.dx = p.dx;
    a.ds0 = p.ds0;
    const bool lookback = p.scan.schedule == kElemLookback;
    return p.scan.gated ? launch_bwd_gated<true>(a, plan, lookback, stream)
                        : launch_bwd_gated<false>(a, plan, lookback, stream);
}

hipError_t launch_step_elem(bool gated, const float* a, const float* x, float* s, int64_t n, bool aligned16,
                            int num_cus, hipStream_t stream) {
    (void)num_cus;
    const bool vec4 = aligned16 && n % 4 == 0;
    const int64_t lanes = vec4 ? n / 4 : n;
    int64_t blocks = (lanes + kThreads - 1) / kThreads;   // one element (or float4) per lane
    if (blocks > (int64_t{1} << 20)) blocks = int64_t{1} << 20;   // beyond 2^28 lanes: grid-stride
    const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
    if (gated) {
        if (vec4) hipLaunchKernelGGL((step_elem_kernel<true, true>), grid, block, 0, stream, a, x, s, n);
        else hipLaunchKernelGGL((step_elem_kernel<true, false>), grid, block, 0, stream, a, x, s, n);
    } else {
        if (vec4) hipLaunchKernelGGL((step_elem_kernel<false, true>), grid, block, 0, stream, a, x, s, n);
        else hipLaunchKernelGGL((step_elem_kernel<false, false>), grid, block, 0, stream, a, x, s, n);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Allocation-free variant: the look-back scratch in a static device array
// ---------------------------------------------------------------------------
// The tile counter, the error flag and the status words of the look-back live
// in `scratch`, one copy per GPU that loads the library, held until the
// process ends.  In host code `scratch` names a host-side stand-in: its device
// address (per device) comes from hipGetSymbolAddress and is the only form
// ever handed to a kernel or a fill.
namespace {

constexpr size_t kScratchHeaderWords = 32;   // [0] tile counter, [1] error flag, rest unused
constexpr int kMaxNoallocDevices = 64;

static __device__ __align__(256) unsigned long long scratch[kNoallocScratchBytes / sizeof(unsigned long long)];

struct NoallocDevice {
    unsigned long long* ptr = nullptr;       // this device's copy of `scratch`
    bool cleared = false;                    // every word zeroed (epoch tag 0) once
    unsigned int epoch = 0;                  // last epoch tag used
    unsigned long long counter_base = 0;     // tiles taken from the counter so far
};

std::mutex g_noalloc_mu;
NoallocDevice g_noalloc[kMaxNoallocDevices];

}  // namespace

size_t noalloc_words_capacity() { return kNoallocScratchBytes / sizeof(unsigned long long) - kScratchHeaderWords; }

int launch_scan_elem_noalloc(ElemParams p, const ElemPlan& plan, int device, hipStream_t stream) {
    const bool lookback = p.schedule == kElemLookback;
    if (device < 0 || device >= kMaxNoallocDevices) return kNoallocUnsupported;
    if (lookback && plan.words > noalloc_words_capacity()) return kNoallocUnsupported;
    // one lock over set-up, launch and bookkeeping: the counter base of a
    // launch must be the sum of the grids launched before it on this device
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    NoallocDevice& d = g_noalloc[device];
    if (!d.ptr) {
        // set-up, once per device, with that device current (the caller's)
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return kNoallocDevice;
        }
        d.ptr = static_cast<unsigned long long*>(ptr);
    }
    if (lookback) {
        if (!d.cleared || d.epoch == 0xffffffffu) {
            // tags must never repeat without a clear: zero every word (and the
            // counter, whose base restarts at 0) with a fill kernel on the stream
            if (launch_fill_zero_u64(d.ptr, kNoallocScratchBytes / sizeof(unsigned long long), stream) !=
                hipSuccess)
                return kNoallocDevice;
            d.cleared = true;
            d.epoch = 0;
            d.counter_base = 0;
        }
        p.epoch = d.epoch + 1;
        p.counter = d.ptr;
        p.error_flag = reinterpret_cast<unsigned int*>(d.ptr + 1);
        p.words = d.ptr + kScratchHeaderWords;
        p.counter_base = d.counter_base;
    }
    if (launch_scan_elem(p, plan, stream) != hipSuccess) return kNoallocDevice;
    if (lookback) {
        d.epoch = p.epoch;
        d.counter_base += static_cast<unsigned long long>(plan.grid);
    }
    return kNoallocOk;
}

hipError_t launch_fill_zero_u64(unsigned long long* p, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_u64_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, p, n);
    return hipGetLastError();
}

}  // namespace lrs
