/*
 * lrs_abi.h -- C ABI of the linear-recurrence scan library for AMD MI355X
 * (gfx950).  Four scans run on one GPU, asynchronously on a caller's HIP
 * stream:
 *
 *   lrs_scan_fma         s_t = a_t s_{t-1} + b_t                 (per channel)
 *   lrs_scan_gated       s_t = a_t s_{t-1} + (1 - a_t) u_t        (per channel)
 *   lrs_scan_diag_outer  S_t = diag(exp(g_t)) S_{t-1} + (kappa_t k_t) v_t^T,
 *                        o_t = scale S_t^T q_t                     (per head)
 *   lrs_scan_delta       S_t = S_{t-1} + k_t [beta_t (v_t - S_{t-1}^T k_t)]^T,
 *                        o_t = scale S_t^T q_t                     (per head)
 *
 *   lrs_scan_diag_outer_epilogue  as lrs_scan_diag_outer, with a fused output
 *                        epilogue (skip or norm-gate) and fp32 or bf16 output
 *   lrs_scan_diag_outer_keyscale  as lrs_scan_diag_outer, kappa per key
 *   lrs_scan_delta_decay S_t = diag(exp(g_t)) S_{t-1}
 *                            + k_t [beta_t (v_t - S_{t-1}^T k_t)]^T,
 *                        o_t = scale S_t^T q_t                     (per head)
 *
 * plus, for the two elementwise forms, the reverse (gradient) pass
 * (lrs_scan_fma_backward, lrs_scan_gated_backward) and the in-place single
 * step (lrs_step_fma, lrs_step_gated).
 *
 * Every scan takes an initial state and returns the final state, so a long
 * sequence can be processed in segments: running [0,T1) and then [T1,T) with
 * the first call's final state as the second call's initial state gives the
 * same outputs as one run over [0,T) (up to floating-point reassociation).
 *
 * Sources, cited by short name:
 *   [SunnyNet log]  "SunnyNet 工程化实录：一个 O(N) 架构如何长出自己的 C 推理运行时",
 *                   developer.aliyun.com/article/1773847
 *   [vs llama.cpp]  "我拿同一份权重和 llama.cpp 正面比了一场：我手写的 C 内核，慢了 1.1–1.7 倍",
 *                   developer.aliyun.com/article/1775078
 *
 * ABI style follows [SunnyNet log §6]: one symbol prefix, opaque handles,
 * a packed (MAJOR<<16)|(MINOR<<8)|PATCH version checked at load time,
 * capability bits that callers must ignore when unknown, and int32_t status
 * codes and dimensions.
 *
 * Conventions for every scan call
 * -------------------------------
 * Pointers.  All tensor pointers are DEVICE pointers on the context's GPU,
 *   allocated and owned by the caller.  The library never frees them and
 *   keeps no reference after the call returns.  Tensors are dense, row-major,
 *   last axis fastest, with the shapes given per call.  fp32 tensors need
 *   4-byte alignment and bf16 tensors 2-byte alignment; 16-byte alignment
 *   enables the vector paths.  Outputs must not overlap inputs or each other.
 * Dimensions.  int32_t, each >= 1.  Offsets are computed in 64 bits.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *   stream).  Calls only enqueue work and return without synchronizing;
 *   outputs are valid once the stream reaches that point.  A context serves
 *   one stream at a time: its workspace is reused by every call, so calls on
 *   one context must not run concurrently on different streams.  A context is
 *   not thread-safe: calls on one context (lrs_context_set_param included)
 *   must come from one host thread at a time; separate contexts are
 *   independent.
 * Graph capture.  A call may be captured into a HIP graph once the context's
 *   workspace is large enough for it (make one uncaptured call of the same or
 *   a larger size first: growing the workspace allocates and synchronizes).
 *   A captured diag-outer or delta call that would need a larger workspace
 *   returns LRS_E_UNSUPPORTED and captures nothing.  A graph keeps the
 *   workspace it was captured with: once a context has served a captured
 *   call, a later uncaptured call that grows a workspace keeps the old buffer
 *   alive (until lrs_context_destroy) rather than freeing it, so earlier
 *   graphs stay valid.  Destroying the context invalidates every graph that
 *   captured its calls.
 *   Every call keeps no per-call state on the host once captured, so a
 *   replay recomputes it on the captured buffers' current contents.  The
 *   elementwise look-back schedule takes a fresh tile-counter base and
 *   status epoch on the host for every call, which a replay would reuse: an
 *   elementwise call made while its stream is being captured therefore uses
 *   the stream schedule when the schedule is automatic, and returns
 *   LRS_E_UNSUPPORTED (nothing captured) when the look-back is forced.
 * Errors.  Arguments are validated on the host before anything is enqueued.
 *   On LRS_E_INVAL, LRS_E_UNSUPPORTED or LRS_E_NOMEM nothing was enqueued and
 *   the outputs are untouched.  LRS_E_DEVICE means a launch failed; work the
 *   call enqueued before it (clearing a freshly grown workspace) may still run.
 *   LRS_E_INVAL       NULL context or required pointer, a dimension < 1,
 *                     misalignment, an output that overlaps another buffer,
 *                     an unknown mode value.
 *   LRS_E_UNSUPPORTED a dimension above the kernels' limit (documented per
 *                     call), a device that is not gfx950, ABI major mismatch.
 *   LRS_E_NOMEM       the context's workspace could not grow.
 *   LRS_E_DEVICE      the HIP runtime reported an error at launch.
 *   Faults during execution surface at the caller's next synchronization, as
 *   for any HIP kernel.  No C++ exception crosses this ABI; nothing is printed.
 * Numerics.  fp32 state and fp32 outputs.  bf16 inputs are used exactly
 *   (products of bf16 values are exact in fp32); fp32 intermediates that feed
 *   the matrix cores are split into two bf16 terms so their rounding error is
 *   near fp32's.  Results agree with a sequential fp64 evaluation to about
 *   1e-6 (elementwise) and 1e-4 (matrix scans) normwise relative error.
 */
#ifndef LRS_ABI_H
#define LRS_ABI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- version and capabilities [SunnyNet log §6] ------------------------ */
#define LRS_ABI_VERSION_MAJOR 1
#define LRS_ABI_VERSION_MINOR 3
#define LRS_ABI_VERSION_PATCH 0
#define LRS_ABI_VERSION \
    ((LRS_ABI_VERSION_MAJOR << 16) | (LRS_ABI_VERSION_MINOR << 8) | LRS_ABI_VERSION_PATCH)

typedef int32_t lrs_status;
enum {
    LRS_OK = 0,
    LRS_E_INVAL = -1,
    LRS_E_NOMEM = -2,
    LRS_E_IO = -3,          /* reserved, never returned */
    LRS_E_FORMAT = -4,      /* reserved, never returned */
    LRS_E_UNSUPPORTED = -5,
    LRS_E_DEVICE = -6
};

#define LRS_CAP_SCAN_FMA        (1u << 0)
#define LRS_CAP_SCAN_GATED      (1u << 1)
#define LRS_CAP_SCAN_DIAG_OUTER (1u << 2)
#define LRS_CAP_SCAN_DELTA      (1u << 3)
#define LRS_CAP_ELEM_BACKWARD   (1u << 4)   /* since 1.1 */
#define LRS_CAP_ELEM_STEP       (1u << 5)   /* since 1.1 */
#define LRS_CAP_SCAN_DELTA_DECAY (1u << 6)  /* since 1.1 */
#define LRS_CAP_SCAN_DIAG_KEYSCALE (1u << 7) /* since 1.1 */
#define LRS_CAP_SCAN_DIAG_EPILOGUE (1u << 8) /* since 1.1 */
#define LRS_CAP_SCAN_DELTA_OUT  (1u << 9)   /* since 1.2 */

/* Output epilogues and dtypes of lrs_scan_diag_outer_epilogue (since 1.1). */
enum { LRS_EPILOGUE_NONE = 0, LRS_EPILOGUE_SKIP = 1, LRS_EPILOGUE_NORM_GATE = 2 };
enum { LRS_DTYPE_F32 = 0, LRS_DTYPE_BF16 = 1 };

/* Packed version of the library actually loaded. */
uint32_t lrs_abi_version(void);

/* Pass LRS_ABI_VERSION_MAJOR as seen at compile time.  Returns LRS_OK when
 * the loaded library has the same major version, LRS_E_UNSUPPORTED
 * otherwise (the caller must then not use the library). */
lrs_status lrs_abi_check(int32_t caller_major);

/* Bit set of LRS_CAP_*.  Callers must ignore bits they do not know. */
uint32_t lrs_abi_caps(void);

/* Static English description of a status code; never NULL. */
const char* lrs_status_string(lrs_status status);

/* ---- context ------------------------------------------------------------ */
typedef struct LrsContext LrsContext;     /* opaque */
typedef uint16_t lrs_bf16;                /* raw bfloat16 bits */

/* Creates a context bound to HIP device `hip_device`.  The context owns a
 * small device workspace (look-back status words and tile counters) that
 * grows on demand.  Errors: LRS_E_INVAL (out == NULL), LRS_E_UNSUPPORTED (no
 * such device, or not gfx950), LRS_E_NOMEM, LRS_E_DEVICE. */
lrs_status lrs_context_create(int32_t hip_device, LrsContext** out);

/* Synchronizes the device, frees the workspace and the handle.  NULL is a
 * no-op. */
void lrs_context_destroy(LrsContext* ctx);

/* Tuning knobs.  LRS_PARAM_ELEM_SCHEDULE picks how the elementwise scans
 * split the time axis:
 *   LRS_ELEM_SCHEDULE_AUTO      (default) stream when it walks a single
 *                               128-step chunk, or when it has a workgroup for
 *                               every compute unit (B * ceil(N / 64) of them
 *                               with 16-byte aligned N % 4 == 0 channels, else
 *                               B * ceil(N / 16)) and T <= 1024; otherwise
 *                               look-back when the time axis spans at least two
 *                               chunks and its status words fit in 256 MB,
 *                               stream otherwise;
 *   LRS_ELEM_SCHEDULE_STREAM    each workgroup owns a set of channels and
 *                               walks the whole time axis, carrying the state
 *                               on chip (no inter-workgroup traffic);
 *   LRS_ELEM_SCHEDULE_LOOKBACK  each workgroup owns one (channels x time)
 *                               tile and obtains its carry-in from earlier
 *                               tiles by a decoupled look-back.
 * Both give results within the documented tolerance of each other.
 *
 * LRS_PARAM_DIAG_SEGMENTS sets how many segments lrs_scan_diag_outer splits
 * the time axis into (each a run of 64-step chunks processed by its own
 * workgroups; a first pass reduces every segment but the last to a decay
 * product and a state contribution, kept in the context's workspace, and a
 * prefix over them gives each segment its starting state):
 *   0 (default)  one workgroup per resident workgroup slot of the device
 *                where a compute unit holds one of them (at least 2 chunks,
 *                128 steps, per segment), about two where it holds more (at
 *                least 4 chunks, 256 steps, per segment);
 *   n >= 1       n segments (capped at the number of chunks).
 * Any value gives results within the documented tolerance.
 *
 * LRS_PARAM_DELTA_SEGMENTS (since 1.3) sets how many time segments the delta
 * rule calls (lrs_scan_delta, lrs_scan_delta_decay, lrs_scan_delta_out) split
 * the chunks into.  A segment pass gives each segment but the last its
 * transition S_out = A_s S_in + B_s (A_s from identity columns run through
 * the same update with zero values), a prefix over them gives each segment
 * its starting state, and the output pass runs every segment at once; the
 * context keeps the states and transitions (4 K (K + 2V) bytes per (batch,
 * head) and segment) beside the per-chunk workspace:
 *   0 (default)  one segment while the (batch, head, 16-column V-tile)
 *                workgroups outnumber half the compute units; otherwise the
 *                most segments (of at least 8 chunks, 512 steps) whose output
 *                pass and segment pass each still fit the compute units once;
 *   1            one pass over all chunks;
 *   n >= 2       n segments (capped at the number of chunks).
 * Any value gives results within the documented tolerance.
 *
 * LRS_PARAM_LOOKBACK_DELAY_SEED (since 1.2) is a verification knob for the
 * elementwise look-back schedule (forward scans and gradient passes):
 *   0 (default)  off;
 *   n >= 1       every look-back tile sleeps a pseudo-random time seeded by n
 *                (0 to about 4 us, per tile) before it publishes its aggregate,
 *                before it walks back over its predecessors and before it
 *                publishes its inclusive prefix, so tiles reach the status
 *                words in an order unrelated to normal timing.  Results stay
 *                within the documented tolerance; calls are much slower.
 * Errors: LRS_E_INVAL for a NULL context, unknown parameter or value. */
enum {
    LRS_PARAM_ELEM_SCHEDULE = 1,
    LRS_PARAM_DIAG_SEGMENTS = 2,
    LRS_PARAM_LOOKBACK_DELAY_SEED = 3,
    LRS_PARAM_DELTA_SEGMENTS = 4
};
enum {
    LRS_ELEM_SCHEDULE_AUTO = 0,
    LRS_ELEM_SCHEDULE_STREAM = 1,
    LRS_ELEM_SCHEDULE_LOOKBACK = 2
};
lrs_status lrs_context_set_param(LrsContext* ctx, int32_t param, int32_t value);

/* Waits for all work this context enqueued, then reports whether a kernel
 * gave up a look-back wait (a bounded spin that should never expire; when it
 * does, the affected outputs are NaN).  Returns LRS_OK, LRS_E_DEVICE (a
 * timed-out wait or a HIP error), or LRS_E_INVAL (NULL context).  Clears the
 * flag. */
lrs_status lrs_context_check(LrsContext* ctx);

/* ---- elementwise first-order scans -------------------------------------
 * [SunnyNet log §2.1]: the unified kernel's two forms.
 *
 *   a, b (or u)   fp32 [B,T,N]   inputs, channel (b,n), time t
 *   s0            fp32 [B,N]     initial state; NULL means zeros
 *   s             fp32 [B,T,N]   output: s[:,t-1,:] = s_t, t = 1..T
 *   s_final       fp32 [B,N]     output: s_T (bit-equal to s[:,T-1,:])
 *
 * The gated form is evaluated as written, fma(a, s, (1 - a) u) in fp32 (so a
 * gate of exactly 1 holds the state bit for bit and one of 0 copies u).  Any
 * int32 sizes are accepted (offsets are 64-bit).  The
 * look-back schedule keeps 24 bytes of status words per channel and 128 time
 * steps in the context workspace (about 50 MB for B=16, T=8192, N=2048).
 */
lrs_status lrs_scan_fma(LrsContext* ctx, const float* a, const float* b, const float* s0,
                        float* s, float* s_final, int32_t B, int32_t T, int32_t N,
                        void* stream);

lrs_status lrs_scan_gated(LrsContext* ctx, const float* a, const float* u, const float* s0,
                          float* s, float* s_final, int32_t B, int32_t T, int32_t N,
                          void* stream);

/* ---- reverse (gradient) pass of the elementwise scans -------------------
 * The back-ends' reverse-scan entry [SunnyNet log §8], read as the gradient
 * pass that training needs.  Given the forward call's inputs and states and
 * the gradient of a loss with respect to its outputs, returns the gradients
 * with respect to its inputs.  With gs_t the total gradient reaching s_t,
 *
 *   gs_T = ds_T + ds_final,    gs_t = ds_t + a_{t+1} gs_{t+1}   (t < T)
 *   FMA form:    da_t = gs_t s_{t-1},           db_t = gs_t
 *   gated form:  da_t = gs_t (s_{t-1} - u_t),    du_t = gs_t (1 - a_t)
 *   ds0 = a_1 gs_1,                             s_0 = s0
 *
 *   a, u          fp32 [B,T,N]   the forward inputs (u: gated form only)
 *   s0            fp32 [B,N]     the forward initial state; NULL means zeros
 *   s             fp32 [B,T,N]   the forward states (s[:,t-1,:] = s_t)
 *   ds            fp32 [B,T,N]   gradient with respect to s
 *   ds_final      fp32 [B,N]     gradient with respect to s_final; NULL means zeros
 *   da, db (du)   fp32 [B,T,N]   outputs
 *   ds0           fp32 [B,N]     output; NULL skips it
 *
 * One pass over the data: a, ds and s (and u) are read once and da, db (du)
 * written once, 20 (24) bytes per element.  The gradient recursion runs as a
 * scan over reversed time with the same chunking and look-back as the
 * forward scans (and the same context workspace); errors, limits and
 * alignment rules are those of lrs_scan_fma.
 */
lrs_status lrs_scan_fma_backward(LrsContext* ctx, const float* a, const float* s0,
                                 const float* s, const float* ds, const float* ds_final,
                                 float* da, float* db, float* ds0, int32_t B, int32_t T,
                                 int32_t N, void* stream);

lrs_status lrs_scan_gated_backward(LrsContext* ctx, const float* a, const float* u,
                                   const float* s0, const float* s, const float* ds,
                                   const float* ds_final, float* da, float* du, float* ds0,
                                   int32_t B, int32_t T, int32_t N, void* stream);

/* ---- single step of the elementwise scans --------------------------------
 * The back-ends' single-step entry [SunnyNet log §8]: one time step for every
 * channel, updating the state in place (decode).  A single-sequence step is
 * tiny and costs mostly call overhead [SunnyNet log §2.4], so one call should
 * carry every channel of every sequence and layer that steps together.
 *
 *   a, b (or u)   fp32 [B,N]   this step's inputs
 *   s             fp32 [B,N]   state, read and overwritten:
 *                              s = a s + b   or   s = a s + (1 - a) u
 *
 * Bit-identical to lrs_scan_fma / lrs_scan_gated with T = 1.  s must not
 * overlap a or b (u).  Errors as lrs_scan_fma.
 */
lrs_status lrs_step_fma(LrsContext* ctx, const float* a, const float* b, float* s, int32_t B,
                        int32_t N, void* stream);

lrs_status lrs_step_gated(LrsContext* ctx, const float* a, const float* u, float* s, int32_t B,
                          int32_t N, void* stream);

/* ---- decay-separable outer-product state scan ---------------------------
 * Mamba-2 [SunnyNet log §4.1]: one decay exp(dt*A) per head and step shared by
 * the whole state, injection (dt*B) outer x, readout against C.
 * GLA [SunnyNet log §4.3]: per-key decay diag(exp(gk)), injection k outer v,
 * readout scale * S^T q with scale = K^-1/2.  Both restated in
 * [vs llama.cpp §3].  Per head h (group grp = h / (H/Hg)) and step t:
 *
 *   S_t[i][j] = exp(g_t[i]) S_{t-1}[i][j] + kappa_t k_t[i] v_t[j]
 *   o_t[j]    = scale * sum_i S_t[i][j] q_t[i]        (read after the update)
 *
 *   q, k      bf16 [B,T,Hg,K]    readout and injection key vectors (per group)
 *   v         bf16 [B,T,H,V]     injected value vectors
 *   g         fp32 [B,T,H]       decay_mode 0: log-decay shared by all keys
 *             fp32 [B,T,H,K]     decay_mode 1: log-decay per key
 *   k_scale   fp32 [B,T,H]       kappa_t; NULL means 1
 *   scale     readout scale
 *   s0        fp32 [B,H,K,V]     initial state; NULL means zeros
 *   o         fp32 [B,T,H,V]     output
 *   s_final   fp32 [B,H,K,V]     output: S_T
 *
 * g is a log-decay and is expected to be <= 0 (decay factors in (0,1]); any
 * finite value is accepted.  Limits: 1 <= K <= 128 (LRS_E_UNSUPPORTED above),
 * H % Hg == 0 (LRS_E_INVAL otherwise), decay_mode in {0,1}.  With more than
 * one time segment (LRS_PARAM_DIAG_SEGMENTS) the context keeps a workspace of
 * (segments - 1) * B * H * (ceil(V/VT)*VT*KP + KP) * 4 bytes, KP = 64 for
 * K <= 64 and 128 otherwise, VT = 64 for V <= 64 and 128 otherwise, grown on
 * demand (LRS_E_NOMEM if that allocation fails); growing it first waits for
 * the whole device, since an earlier call on another stream may still use
 * the old workspace.  LRS_E_UNSUPPORTED also when B * H * ceil(V/VT) is
 * 2^27 or more (launch grid limits).
 */
lrs_status lrs_scan_diag_outer(LrsContext* ctx, const lrs_bf16* q, const lrs_bf16* k,
                               const lrs_bf16* v, const float* g, int32_t decay_mode,
                               const float* k_scale, float scale, const float* s0, float* o,
                               float* s_final, int32_t B, int32_t T, int32_t H, int32_t Hg,
                               int32_t K, int32_t V, void* stream);

/* ---- delta-rule state scan ---------------------------------------------
 * DeltaNet [SunnyNet log §4.2], restated in [vs llama.cpp §3].  Per head h
 * and step t:
 *
 *   delta_t = beta_t (v_t - S_{t-1}^T k_t)
 *   S_t     = S_{t-1} + k_t delta_t^T         (= (I - beta k k^T) S + beta k v^T)
 *   o_t     = scale S_t^T q_t                 (the pages use scale = 1)
 *
 *   q, k      bf16 [B,T,H,K]
 *   v         bf16 [B,T,H,V]
 *   beta      fp32 [B,T,H]
 *   s0        fp32 [B,H,K,V]     NULL means zeros
 *   o         fp32 [B,T,H,V]     output
 *   s_final   fp32 [B,H,K,V]     output
 *
 * Limits: 1 <= K <= 128; T <= 4194240 for K <= 64 and T <= 2796160 for
 * K > 64 (LRS_E_UNSUPPORTED beyond: one (batch, head) slice of the workspace
 * must stay under 2 GiB).  The context keeps a workspace per (batch, head,
 * 64-step chunk) of 32 KiB (K <= 64) or 48 KiB (K > 64), holding the chunk's
 * output and state-update factors (plus, when the call runs in time
 * segments, see LRS_PARAM_DELTA_SEGMENTS, their states and transitions),
 * grown on demand (LRS_E_NOMEM if that
 * allocation fails); growing it first waits for the whole device, since an
 * earlier call on another stream may still use the old workspace.
 */
lrs_status lrs_scan_delta(LrsContext* ctx, const lrs_bf16* q, const lrs_bf16* k,
                          const lrs_bf16* v, const float* beta, float scale, const float* s0,
                          float* o, float* s_final, int32_t B, int32_t T, int32_t H, int32_t K,
                          int32_t V, void* stream);

/* ---- decay-separable scan with a fused output epilogue -------------------
 * lrs_scan_diag_outer whose outputs go through an epilogue inside the kernel
 * before they are written, in fp32 or bf16:
 *
 *   LRS_EPILOGUE_NONE       out = o
 *   LRS_EPILOGUE_SKIP       out = o + d_skip[h] * v          (Mamba-2's D x skip)
 *   LRS_EPILOGUE_NORM_GATE  out = o / sqrt(mean_j o_j^2 + eps) * norm_weight * silu(gate)
 *                           (GLA's output norm and gate [SunnyNet log §4.3]:
 *                           RMSNorm over the value axis of each head, then the gate)
 *
 * with o = scale S_t^T q_t as in lrs_scan_diag_outer and silu(x) = x / (1 + e^-x).
 *
 *   d_skip       fp32 [H]          SKIP only (else ignored)
 *   gate         bf16 [B,T,H,V]    NORM_GATE only
 *   norm_weight  fp32 [V]          NORM_GATE only; NULL means ones
 *   eps          >= 0              NORM_GATE only
 *   out_dtype    LRS_DTYPE_F32 or LRS_DTYPE_BF16 (rounded to nearest even)
 *   o            [B,T,H,V] of out_dtype (device pointer, 4- or 2-byte aligned)
 *
 * Writing bf16 halves the output bytes, which are 28-61% of these scans'
 * traffic.  NORM_GATE needs V <= 128 (LRS_E_UNSUPPORTED above).  Other
 * arguments, limits and errors as lrs_scan_diag_outer.
 */
lrs_status lrs_scan_diag_outer_epilogue(LrsContext* ctx, const lrs_bf16* q, const lrs_bf16* k,
                                        const lrs_bf16* v, const float* g, int32_t decay_mode,
                                        const float* k_scale, float scale, const float* s0,
                                        int32_t epilogue, const float* d_skip, const lrs_bf16* gate,
                                        const float* norm_weight, float eps, int32_t out_dtype,
                                        void* o, float* s_final, int32_t B, int32_t T, int32_t H,
                                        int32_t Hg, int32_t K, int32_t V, void* stream);

/* ---- decay-separable scan with a per-key injection scale ------------------
 * As lrs_scan_diag_outer with a per-key decay (decay mode 1), but kappa is a
 * vector over the keys:
 *
 *   S_t[i][j] = exp(g_t[i]) S_{t-1}[i][j] + kappa_t[i] k_t[i] v_t[j],
 *   o_t = scale S_t^T q_t
 *
 * The matrix associative memory [vs llama.cpp §8],
 * S_t = p (.) S_{t-1} + (1 - p) (.) (v_t (x) k_t) with p on the key axis, is
 * this call with g = log p and kappa = 1 - p (its output projection is a
 * model layer and stays with the caller).
 *
 *   q, k     bf16 [B,T,Hg,K];  v bf16 [B,T,H,V]
 *   g        fp32 [B,T,H,K]    log-decay per key
 *   k_scale  fp32 [B,T,H,K]    kappa per key, required
 *   s0, o, s_final as lrs_scan_diag_outer
 *
 * Limits, workspace and errors as lrs_scan_diag_outer (decay mode 1).
 */
lrs_status lrs_scan_diag_outer_keyscale(LrsContext* ctx, const lrs_bf16* q, const lrs_bf16* k,
                                        const lrs_bf16* v, const float* g, const float* k_scale,
                                        float scale, const float* s0, float* o, float* s_final,
                                        int32_t B, int32_t T, int32_t H, int32_t Hg, int32_t K,
                                        int32_t V, void* stream);

/* ---- delta rule with a per-key decay --------------------------------------
 * RWKV-7's state update [SunnyNet log §5.1], which the page writes for a
 * value-major state as S (.) w - (S k) k^T + v k^T.  Here the state is
 * key-major ([K,V], as in lrs_scan_delta) and the write carries the in-context
 * rate beta_t (beta = 1 is the page's form):
 *
 *   S_t = (diag(w_t) - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   w_t = exp(g_t)
 *   o_t = scale S_t^T q_t
 *
 * The removal reads the state before the decay.  With g = 0 this is
 * lrs_scan_delta.
 *
 *   q, k       bf16 [B,T,H,K]
 *   v          bf16 [B,T,H,V]
 *   g          fp32 [B,T,H,K]   log-decay per key (w = exp(g)), required
 *   beta       fp32 [B,T,H]
 *   s0         fp32 [B,H,K,V]   NULL means zeros
 *   o          fp32 [B,T,H,V]   output
 *   s_final    fp32 [B,H,K,V]   output
 *
 * Limits: 1 <= K <= 128; T <= 2088960 for K <= 64 and T <= 1193024 for
 * K > 64 (LRS_E_UNSUPPORTED beyond).  The context workspace holds 64.25 KiB
 * (K <= 64) or 112.5 KiB (K > 64) per (b,h,64-step chunk): the factors of
 * lrs_scan_delta plus the chunk's decayed keys and queries and its total
 * decay, grown on demand as for lrs_scan_delta.  Any finite g is accepted; chunks in which some key's
 * running log-decay spans more than 60 nats take a slower exact path.
 * Errors as lrs_scan_delta.
 */
lrs_status lrs_scan_delta_decay(LrsContext* ctx, const lrs_bf16* q, const lrs_bf16* k,
                                const lrs_bf16* v, const float* g, const float* beta, float scale,
                                const float* s0, float* o, float* s_final, int32_t B, int32_t T,
                                int32_t H, int32_t K, int32_t V, void* stream);

/* ---- delta rule with an fp32 or bf16 output (since 1.2) --------------------
 * lrs_scan_delta (g == NULL) or lrs_scan_delta_decay (g != NULL) with the
 * output written as out_dtype: LRS_DTYPE_F32, or LRS_DTYPE_BF16 rounded to
 * nearest even from the fp32 result.  DeltaNet's update and readout
 * [SunnyNet log §4.2]; the per-key decay of RWKV-7 [SunnyNet log §5.1].
 *
 *   g          fp32 [B,T,H,K] per-key log-decay, or NULL for the plain delta rule
 *   out_dtype  LRS_DTYPE_F32 or LRS_DTYPE_BF16
 *   o          [B,T,H,V] of out_dtype (device pointer, 4- or 2-byte aligned)
 *
 * The state stays fp32 (s0, s_final).  A bf16 o halves the output bytes, the
 * largest single term of these scans' traffic (39% of the DeltaNet
 * workload's at fp32).  Other arguments, limits, workspace and errors as
 * lrs_scan_delta (g == NULL) or lrs_scan_delta_decay.
 */
lrs_status lrs_scan_delta_out(LrsContext* ctx, const lrs_bf16* q, const lrs_bf16* k, const lrs_bf16* v,
                              const float* g, const float* beta, float scale, const float* s0,
                              int32_t out_dtype, void* o, float* s_final, int32_t B, int32_t T, int32_t H,
                              int32_t K, int32_t V, void* stream);

/* ---- allocation-free gated scan (since 1.2) --------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * scan as lrs_scan_gated ([SunnyNet log §2.1]), without a context: it runs on
 * the calling thread's current HIP device and calls no hipMalloc, hipFree or
 * other allocating routine.  Its look-back scratch (tile counter, error flag
 * and status words) is a static device array of 64 MiB that the library holds
 * on each GPU it runs on until the process ends.
 *
 *   a, u, s0, s, s_final   as lrs_scan_gated (s0 may be NULL)
 *
 * Limit: the look-back needs 24 bytes per channel and 128-step chunk (32-step
 * chunks below T = 512); when the time axis spans two or more chunks those
 * words must fit in the scratch, 64 MiB - 256 B (e.g. B=16, T=8192, N=2048
 * needs 48 MiB).  Larger shapes return LRS_E_UNSUPPORTED before anything is
 * enqueued or any HIP call is made.  Under graph capture the call takes the
 * stream schedule, which uses no scratch.
 * Every call on one GPU shares that GPU's scratch (the status words carry a
 * per-call tag, so nothing needs clearing between calls; the library zeroes
 * the array with a fill kernel on its first use on a device).  Calls that
 * overlap on one GPU -- on different streams, or from threads that do not
 * order their streams -- race on it and give wrong results; calls issued one
 * after another on one stream are safe from any thread.  A look-back wait
 * that expires (it should never) leaves NaN outputs; there is no context to
 * report it.  Errors as lrs_scan_gated, plus LRS_E_DEVICE when no HIP device
 * is current.
 */
lrs_status lrs_scan_gated_noalloc(const float* a, const float* u, const float* s0, float* s,
                                  float* s_final, int32_t B, int32_t T, int32_t N, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LRS_ABI_H */
