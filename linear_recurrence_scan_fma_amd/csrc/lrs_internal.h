// Internal interface between the C-ABI layer (abi.cpp) and the HIP kernels.
// Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace lrs {

// ---------------------------------------------------------------------------
// Elementwise first-order scans (FMA and gated forms).
// ---------------------------------------------------------------------------
enum ElemSchedule : int { kElemStream = 1, kElemLookback = 2 };

struct ElemParams {
    const float* a;
    const float* x;      // b (FMA form) or u (gated form)
    const float* s0;     // nullable
    float* s;
    float* s_final;
    int64_t B, T, N;
    bool gated;
    int schedule;        // kElemStream or kElemLookback (already resolved)
    // look-back workspace (schedule == kElemLookback only)
    unsigned long long* words;    // status words, elem_lookback_words() of them
    unsigned long long* counter;  // monotonically increasing tile counter
    unsigned long long counter_base;
    unsigned int epoch;           // tag of this call's status words, never 0
    unsigned int* error_flag;     // set to 1 when a bounded wait expires
    unsigned int delay_seed;      // nonzero: the scrambled-arrival look-back variant
};

struct ElemPlan {
    int vec;            // channels per lane (4 or 1)
    int rows;           // rows per lane per chunk
    int64_t chan_tiles; // channel tiles per batch row
    int64_t chunks;     // time chunks
    int64_t grid;       // workgroups launched
    size_t words;       // status words needed (look-back only)
};

// Resolves vector width, chunk shape and grid for a schedule.
ElemPlan elem_plan(int64_t B, int64_t T, int64_t N, bool aligned16, int schedule);
// Picks a schedule for a shape when the caller asked for "auto".
int elem_auto_schedule(int64_t B, int64_t T, int64_t N, bool aligned16, int num_cus);
hipError_t launch_scan_elem(const ElemParams& p, const ElemPlan& plan, hipStream_t stream);

// Reverse (gradient) pass of an elementwise scan: the reversed FMA scan of the
// incoming gradients, fused with the input gradients.  `scan` carries the
// shape, form (gated), schedule and look-back state; scan.s0 is the gradient
// of the final state (nullable) and scan.a/x/s/s_final are unused.  The plan
// is elem_plan() of the same shape.
struct ElemBwdParams {
    ElemParams scan;
    const float* a;
    const float* u;      // gated form only
    const float* s0;     // forward initial state, nullable
    const float* s;      // forward states
    const float* ds;
    float* da;
    float* dx;           // db (FMA form) or du (gated form)
    float* ds0;          // nullable
};
hipError_t launch_scan_elem_bwd(const ElemBwdParams& p, const ElemPlan& plan, hipStream_t stream);

// Allocation-free variant of launch_scan_elem: the look-back scratch (tile
// counter, error flag, status words) is a static device array of
// kNoallocScratchBytes per GPU.  Resolves this device's copy on its first use
// (hipGetSymbolAddress with the device current), takes the look-back epoch
// and counter base from per-device host state, launches, and advances that
// state, all under one lock.  `p` carries the shape, form and resolved
// schedule; its look-back fields are filled here.  Returns a kNoalloc* code.
constexpr size_t kNoallocScratchBytes = size_t{64} << 20;
enum NoallocStatus : int { kNoallocOk = 0, kNoallocUnsupported = 1, kNoallocDevice = 2 };
// Status words the scratch holds (the look-back limit of the variant).
size_t noalloc_words_capacity();
int launch_scan_elem_noalloc(ElemParams p, const ElemPlan& plan, int device, hipStream_t stream);

// One in-place step s = a s + x (or the gated form) over n channels.
hipError_t launch_step_elem(bool gated, const float* a, const float* x, float* s, int64_t n, bool aligned16,
                            int num_cus, hipStream_t stream);

// ---------------------------------------------------------------------------
// Decay-separable outer-product state scan.
// ---------------------------------------------------------------------------
struct DiagParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* g;
    int decay_mode;        // 0: g [B,T,H]; 1: g [B,T,H,K]
    const float* k_scale;  // nullable; [B,T,H], or [B,T,H,K] with k_scale_key
    int k_scale_key;       // kappa per key (decay mode 1 only)
    float scale;
    const float* s0;       // nullable
    float* o;              // fp32, or bf16 when out_bf16
    float* s_final;
    int B, T, H, Hg, K, V;
    int vec;               // 16-byte vector loads and stores allowed
    // output epilogue: 0 none, 1 o + D_h v, 2 RMSNorm(o) * norm_w * silu(gate) (needs V <= 128)
    int epi_kind;
    int out_bf16;
    const float* d_skip;       // [H]
    const uint16_t* gate;      // bf16 [B,T,H,V]
    const float* norm_w;       // [V], nullable
    float eps;
};

// Time-axis split of the diag-outer scan: chunks of 64 steps grouped into
// segments; a segment count above one needs diag_outer_workspace_bytes().
struct DiagPlan {
    int waves;             // waves per workgroup (16 state columns each)
    int nchunks;
    int vtiles;
    int nseg;
    int cps;               // chunks per segment
};

// requested_segments <= 0 picks as many segments as fill the chip's resident
// workgroup slots once.
DiagPlan diag_outer_plan(int B, int T, int H, int V, int K, int decay_mode, bool kscale_key, bool vec,
                         int num_cus, int requested_segments);
size_t diag_outer_workspace_bytes(int B, int H, int K, int V, int nseg);
hipError_t launch_scan_diag_outer(const DiagParams& p, const DiagPlan& plan, void* workspace,
                                  hipStream_t stream);

// ---------------------------------------------------------------------------
// Delta-rule state scan.
// ---------------------------------------------------------------------------
struct DeltaParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* beta;
    const float* g;        // per-key log-decay [B,T,H,K]; NULL: the plain delta rule
    float scale;
    const float* s0;       // nullable
    float* o;
    float* s_final;
    int B, T, H, K, V;
    int vec;               // 16-byte vector loads allowed
    int out_bf16;          // o is bf16 (round to nearest even) instead of fp32
    int nseg;              // time segments (<= 1: one pass over all chunks)
};

int delta_vtile();
// Largest K of the decayed form.
int delta_decay_max_k();
// Device workspace the delta scan needs: per-chunk UT-transform planes (plus
// the decayed operands with a decay), and with nseg > 1 the segment states and
// transitions.
size_t delta_chunk_workspace_bytes(int B, int T, int H, int K, bool decay);
size_t delta_workspace_bytes(int B, int T, int H, int K, int V, bool decay, int nseg);
// Time segments for a call: `requested` > 0 forces a count (capped at the
// chunk count), else the automatic choice for `num_cus` compute units.
int delta_plan_segments(int B, int T, int H, int K, int V, int num_cus, int requested);
hipError_t launch_scan_delta(const DeltaParams& p, void* workspace, hipStream_t stream);

// Fills `n` 64-bit words with zero (used to reset look-back status words).
hipError_t launch_fill_zero_u64(unsigned long long* p, size_t n, hipStream_t stream);

}  // namespace lrs
