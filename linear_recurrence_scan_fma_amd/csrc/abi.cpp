// C-ABI layer: argument validation, the opaque context and its workspace,
// and kernel launches.  Declarations and the contract live in include/lrs_abi.h.
//
// ABI style after [SunnyNet log §6] ("SunnyNet 工程化实录：一个 O(N) 架构如何长出自己的
// C 推理运行时", developer.aliyun.com/article/1773847): prefixed symbols, opaque
// handles, packed version, capability bits, int32 status codes and dims.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "lrs_abi.h"
#include "lrs_internal.h"

#define LRS_API extern "C" __attribute__((visibility("default")))

struct LrsContext {
    int device = 0;
    int num_cus = 256;
    int elem_schedule = LRS_ELEM_SCHEDULE_AUTO;
    unsigned int lookback_delay_seed = 0;   // LRS_PARAM_LOOKBACK_DELAY_SEED
    // small fixed block: [0] tile counter (u64), [1] error flag (u32 in a u64 slot)
    unsigned long long* fixed = nullptr;
    // look-back status words, grown on demand
    unsigned long long* words = nullptr;
    size_t words_cap = 0;
    unsigned int epoch = 0;                 // last epoch used; status words hold 0 initially
    unsigned long long counter_base = 0;    // tiles taken from the counter so far
    // delta-rule scratch (per-chunk UT-transform planes), grown on demand
    void* delta_ws = nullptr;
    size_t delta_ws_bytes = 0;
    // diag-outer segment pairs (decay products and state contributions), grown on demand
    int diag_segments = 0;   // 0: automatic
    int delta_segments = 0;  // 0: automatic
    void* diag_ws = nullptr;
    size_t diag_ws_bytes = 0;
    hipStream_t last_stream = nullptr;
    bool used = false;
    // Set once a diag-outer or delta call has been captured into a HIP graph:
    // such a graph keeps the workspace pointer it was captured with, so from
    // then on a grown workspace's old buffer is retired (kept until
    // lrs_context_destroy) instead of freed.
    bool captured = false;
    std::vector<void*> retired;
};

namespace {

// Keeps the caller's current device unchanged across a call.
class DeviceGuard {
   public:
    explicit DeviceGuard(int dev) {
        ok_ = hipGetDevice(&prev_) == hipSuccess;
        if (ok_ && prev_ != dev) ok_ = hipSetDevice(dev) == hipSuccess;
        else if (ok_) prev_ = -1;
    }
    ~DeviceGuard() {
        if (prev_ >= 0) (void)hipSetDevice(prev_);
    }
    bool ok() const { return ok_; }

   private:
    int prev_ = -1;
    bool ok_ = false;
};

struct Span {
    const void* p;
    size_t bytes;
};

bool overlaps(const Span& x, const Span& y) {
    if (!x.p || !y.p || x.bytes == 0 || y.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(x.p), a1 = a0 + x.bytes;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(y.p), b1 = b0 + y.bytes;
    return a0 < b1 && b0 < a1;
}

// Every output must be disjoint from every other buffer.
bool outputs_disjoint(const Span* outs, int nout, const Span* ins, int nin) {
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlaps(outs[i], ins[j])) return false;
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(outs[i], outs[j])) return false;
    }
    return true;
}

bool aligned(const void* p, size_t a) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % a == 0; }

bool mul_ok(int64_t& acc, int64_t v) {
    if (v <= 0) return false;
    if (acc > INT64_MAX / v) return false;
    acc *= v;
    return true;
}

// True while `stream` is being captured into a graph.
bool capturing(hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(stream, &cs) == hipSuccess && cs == hipStreamCaptureStatusActive;
}

// Growing a context buffer frees the old one: every stream may still hold work
// of an earlier call that uses it (a context serves one stream at a time, but
// successive calls may use different streams), so the whole device is waited
// for first.  Growth is rare: a context keeps its largest size.
lrs_status grow_words(LrsContext* ctx, size_t need, hipStream_t stream) {
    if (need <= ctx->words_cap) return LRS_OK;
    size_t cap = ctx->words_cap ? ctx->words_cap : 4096;
    while (cap < need) cap *= 2;
    if (ctx->words) {
        if (hipDeviceSynchronize() != hipSuccess) return LRS_E_DEVICE;
        (void)hipFree(ctx->words);
        ctx->words = nullptr;
        ctx->words_cap = 0;
    }
    void* p = nullptr;
    if (hipMalloc(&p, cap * sizeof(unsigned long long)) != hipSuccess) {
        (void)hipGetLastError();
        return LRS_E_NOMEM;
    }
    ctx->words = static_cast<unsigned long long*>(p);
    ctx->words_cap = cap;
    if (lrs::launch_fill_zero_u64(ctx->words, cap, stream) != hipSuccess) return LRS_E_DEVICE;
    ctx->epoch = 0;  // fresh words hold tag 0; the next epoch is 1
    return LRS_OK;
}

// Next epoch tag for look-back status words; tags are never 0 and never reused
// without clearing the words first.
lrs_status next_epoch(LrsContext* ctx, hipStream_t stream, unsigned int* out) {
    if (ctx->epoch == 0xffffffffu) {
        if (lrs::launch_fill_zero_u64(ctx->words, ctx->words_cap, stream) != hipSuccess)
            return LRS_E_DEVICE;
        ctx->epoch = 0;
    }
    *out = ++ctx->epoch;
    return LRS_OK;
}

// Compute units of `device` (an attribute query, no allocation), asked once per
// device; threads may race on the first query, which only repeats it.
int device_cus(int device) {
    constexpr int kDevices = 64;
    static std::atomic<int> cached[kDevices];
    if (device < 0 || device >= kDevices) return 256;
    int n = cached[device].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cached[device].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Resolves the schedule and plan of an elementwise pass over [B,T,N] and, for
// the look-back schedule, sizes the status words and takes a fresh epoch.
// Fills p.B/T/N, p.gated, p.schedule and the look-back fields.  A look-back
// launch carries its tile-counter base and status epoch from the host, which
// a graph replay would reuse, so a call captured into a graph uses the stream
// schedule (automatic choice) or is refused (look-back forced).
lrs_status elem_prepare(LrsContext* ctx, bool gated, int32_t B, int32_t T, int32_t N, bool al16,
                        hipStream_t stream, lrs::ElemPlan& plan, lrs::ElemParams& p) {
    // The capture query runs only where a look-back could be chosen: a short
    // call (one chunk) or a forced stream schedule pays no runtime query.
    int schedule = ctx->elem_schedule;
    if (schedule == LRS_ELEM_SCHEDULE_LOOKBACK && capturing(stream)) return LRS_E_UNSUPPORTED;
    if (schedule == LRS_ELEM_SCHEDULE_AUTO) {
        schedule = lrs::elem_auto_schedule(B, T, N, al16, ctx->num_cus) == lrs::kElemLookback
                       ? LRS_ELEM_SCHEDULE_LOOKBACK : LRS_ELEM_SCHEDULE_STREAM;
        if (schedule == LRS_ELEM_SCHEDULE_LOOKBACK && capturing(stream)) schedule = LRS_ELEM_SCHEDULE_STREAM;
    }
    const int ksched = schedule == LRS_ELEM_SCHEDULE_LOOKBACK ? lrs::kElemLookback : lrs::kElemStream;
    plan = lrs::elem_plan(B, T, N, al16, ksched);
    if (plan.grid > 0x7fffffff) return LRS_E_UNSUPPORTED;
    p.B = B;
    p.T = T;
    p.N = N;
    p.gated = gated;
    p.schedule = ksched;
    if (ksched == lrs::kElemLookback) {
        lrs_status st = grow_words(ctx, plan.words, stream);
        if (st != LRS_OK) return st;
        st = next_epoch(ctx, stream, &p.epoch);
        if (st != LRS_OK) return st;
        p.words = ctx->words;
        p.counter = ctx->fixed;
        p.counter_base = ctx->counter_base;
        p.error_flag = reinterpret_cast<unsigned int*>(ctx->fixed + 1);
        p.delay_seed = ctx->lookback_delay_seed;
    }
    return LRS_OK;
}

// Bookkeeping after a successful elementwise launch.
void elem_launched(LrsContext* ctx, const lrs::ElemPlan& plan, const lrs::ElemParams& p,
                   hipStream_t stream) {
    if (p.schedule == lrs::kElemLookback) ctx->counter_base += static_cast<unsigned long long>(plan.grid);
    ctx->last_stream = stream;
    ctx->used = true;
}

// Shared size checks of the elementwise calls: dims >= 1 and B*T*N*8 bytes
// representable.  Returns the element count in `seq`.
bool elem_dims_ok(int32_t B, int32_t T, int32_t N, int64_t& seq) {
    if (B < 1 || T < 1 || N < 1) return false;
    seq = B;
    return mul_ok(seq, T) && mul_ok(seq, N) && seq <= INT64_MAX / 8;
}

lrs_status scan_elem(LrsContext* ctx, bool gated, const float* a, const float* x,
                     const float* s0, float* s, float* s_final, int32_t B, int32_t T, int32_t N,
                     void* stream_ptr) {
    if (!ctx || !a || !x || !s || !s_final) return LRS_E_INVAL;
    int64_t seq = 0;
    if (!elem_dims_ok(B, T, N, seq)) return LRS_E_INVAL;
    if (!aligned(a, 4) || !aligned(x, 4) || !aligned(s0, 4) || !aligned(s, 4) || !aligned(s_final, 4))
        return LRS_E_INVAL;
    const size_t seq_bytes = static_cast<size_t>(seq) * sizeof(float);
    const size_t st_bytes = static_cast<size_t>(B) * N * sizeof(float);
    const Span ins[] = {{a, seq_bytes}, {x, seq_bytes}, {s0, st_bytes}};
    const Span outs[] = {{s, seq_bytes}, {s_final, st_bytes}};
    if (!outputs_disjoint(outs, 2, ins, 3)) return LRS_E_INVAL;

    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return LRS_E_DEVICE;

    const bool al16 = aligned(a, 16) && aligned(x, 16) && aligned(s, 16);
    lrs::ElemPlan plan{};
    lrs::ElemParams p{};
    const lrs_status st = elem_prepare(ctx, gated, B, T, N, al16, stream, plan, p);
    if (st != LRS_OK) return st;
    p.a = a;
    p.x = x;
    p.s0 = s0;
    p.s = s;
    p.s_final = s_final;
    if (lrs::launch_scan_elem(p, plan, stream) != hipSuccess) return LRS_E_DEVICE;
    elem_launched(ctx, plan, p, stream);
    return LRS_OK;
}

lrs_status scan_elem_bwd(LrsContext* ctx, bool gated, const float* a, const float* u,
                         const float* s0, const float* s, const float* ds, const float* ds_final,
                         float* da, float* dx, float* ds0, int32_t B, int32_t T, int32_t N,
                         void* stream_ptr) {
    if (!ctx || !a || !s || !ds || !da || !dx || (gated && !u)) return LRS_E_INVAL;
    int64_t seq = 0;
    if (!elem_dims_ok(B, T, N, seq)) return LRS_E_INVAL;
    if (!aligned(a, 4) || !aligned(u, 4) || !aligned(s0, 4) || !aligned(s, 4) || !aligned(ds, 4) ||
        !aligned(ds_final, 4) || !aligned(da, 4) || !aligned(dx, 4) || !aligned(ds0, 4))
        return LRS_E_INVAL;
    const size_t seq_bytes = static_cast<size_t>(seq) * sizeof(float);
    const size_t st_bytes = static_cast<size_t>(B) * N * sizeof(float);
    const Span ins[] = {{a, seq_bytes}, {u, seq_bytes}, {s0, st_bytes}, {s, seq_bytes},
                        {ds, seq_bytes}, {ds_final, st_bytes}};
    const Span outs[] = {{da, seq_bytes}, {dx, seq_bytes}, {ds0, st_bytes}};
    if (!outputs_disjoint(outs, 3, ins, 6)) return LRS_E_INVAL;

    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return LRS_E_DEVICE;

    const bool al16 = aligned(a, 16) && aligned(u, 16) && aligned(s, 16) && aligned(ds, 16) &&
                      aligned(da, 16) && aligned(dx, 16);
    lrs::ElemBwdParams p{};
    lrs::ElemPlan plan{};
    const lrs_status st = elem_prepare(ctx, gated, B, T, N, al16, stream, plan, p.scan);
    if (st != LRS_OK) return st;
    p.scan.s0 = ds_final;   // the reversed scan starts from the final state's gradient
    p.a = a;
    p.u = gated ? u : nullptr;
    p.s0 = s0;
    p.s = s;
    p.ds = ds;
    p.da = da;
    p.dx = dx;
    p.ds0 = ds0;
    if (lrs::launch_scan_elem_bwd(p, plan, stream) != hipSuccess) return LRS_E_DEVICE;
    elem_launched(ctx, plan, p.scan, stream);
    return LRS_OK;
}

lrs_status step_elem(LrsContext* ctx, bool gated, const float* a, const float* x, float* s,
                     int32_t B, int32_t N, void* stream_ptr) {
    if (!ctx || !a || !x || !s) return LRS_E_INVAL;
    int64_t n = 0;
    if (!elem_dims_ok(B, 1, N, n)) return LRS_E_INVAL;
    if (!aligned(a, 4) || !aligned(x, 4) || !aligned(s, 4)) return LRS_E_INVAL;
    const size_t bytes = static_cast<size_t>(n) * sizeof(float);
    const Span ins[] = {{a, bytes}, {x, bytes}};
    const Span outs[] = {{s, bytes}};
    if (!outputs_disjoint(outs, 1, ins, 2)) return LRS_E_INVAL;

    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return LRS_E_DEVICE;
    const bool al16 = aligned(a, 16) && aligned(x, 16) && aligned(s, 16);
    if (lrs::launch_step_elem(gated, a, x, s, n, al16, ctx->num_cus, stream) != hipSuccess)
        return LRS_E_DEVICE;
    ctx->last_stream = stream;
    ctx->used = true;
    return LRS_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// version, capabilities, status strings
// ---------------------------------------------------------------------------
LRS_API uint32_t lrs_abi_version(void) { return LRS_ABI_VERSION; }

LRS_API lrs_status lrs_abi_check(int32_t caller_major) {
    return caller_major == LRS_ABI_VERSION_MAJOR ? LRS_OK : LRS_E_UNSUPPORTED;
}

LRS_API uint32_t lrs_abi_caps(void) {
    return LRS_CAP_SCAN_FMA | LRS_CAP_SCAN_GATED | LRS_CAP_SCAN_DIAG_OUTER | LRS_CAP_SCAN_DELTA |
           LRS_CAP_ELEM_BACKWARD | LRS_CAP_ELEM_STEP | LRS_CAP_SCAN_DELTA_DECAY |
           LRS_CAP_SCAN_DIAG_KEYSCALE | LRS_CAP_SCAN_DIAG_EPILOGUE | LRS_CAP_SCAN_DELTA_OUT;
}

LRS_API const char* lrs_status_string(lrs_status status) {
    switch (status) {
        case LRS_OK: return "ok";
        case LRS_E_INVAL: return "invalid argument";
        case LRS_E_NOMEM: return "out of device memory";
        case LRS_E_IO: return "i/o error";
        case LRS_E_FORMAT: return "bad format";
        case LRS_E_UNSUPPORTED: return "unsupported";
        case LRS_E_DEVICE: return "device or runtime error";
        default: return "unknown status";
    }
}

// ---------------------------------------------------------------------------
// context
// ---------------------------------------------------------------------------
LRS_API lrs_status lrs_context_create(int32_t hip_device, LrsContext** out) {
    if (!out) return LRS_E_INVAL;
    *out = nullptr;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || hip_device < 0 || hip_device >= count) {
        (void)hipGetLastError();
        return LRS_E_UNSUPPORTED;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, hip_device) != hipSuccess) return LRS_E_DEVICE;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return LRS_E_UNSUPPORTED;

    DeviceGuard guard(hip_device);
    if (!guard.ok()) return LRS_E_DEVICE;
    LrsContext* ctx = new (std::nothrow) LrsContext();
    if (!ctx) return LRS_E_NOMEM;
    ctx->device = hip_device;
    ctx->num_cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
    void* p = nullptr;
    if (hipMalloc(&p, 256) != hipSuccess) {
        (void)hipGetLastError();
        delete ctx;
        return LRS_E_NOMEM;
    }
    ctx->fixed = static_cast<unsigned long long*>(p);
    if (hipMemset(ctx->fixed, 0, 256) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(ctx->fixed);
        delete ctx;
        return LRS_E_DEVICE;
    }
    *out = ctx;
    return LRS_OK;
}

LRS_API void lrs_context_destroy(LrsContext* ctx) {
    if (!ctx) return;
    {
        DeviceGuard guard(ctx->device);
        (void)hipDeviceSynchronize();
        if (ctx->words) (void)hipFree(ctx->words);
        if (ctx->delta_ws) (void)hipFree(ctx->delta_ws);
        if (ctx->diag_ws) (void)hipFree(ctx->diag_ws);
        if (ctx->fixed) (void)hipFree(ctx->fixed);
        for (void* r : ctx->retired) (void)hipFree(r);
    }
    delete ctx;
}

LRS_API lrs_status lrs_context_set_param(LrsContext* ctx, int32_t param, int32_t value) {
    if (!ctx) return LRS_E_INVAL;
    if (param == LRS_PARAM_ELEM_SCHEDULE) {
        if (value != LRS_ELEM_SCHEDULE_AUTO && value != LRS_ELEM_SCHEDULE_STREAM &&
            value != LRS_ELEM_SCHEDULE_LOOKBACK)
            return LRS_E_INVAL;
        ctx->elem_schedule = value;
        return LRS_OK;
    }
    if (param == LRS_PARAM_DIAG_SEGMENTS) {
        if (value < 0) return LRS_E_INVAL;
        ctx->diag_segments = value;
        return LRS_OK;
    }
    if (param == LRS_PARAM_DELTA_SEGMENTS) {
        if (value < 0) return LRS_E_INVAL;
        ctx->delta_segments = value;
        return LRS_OK;
    }
    if (param == LRS_PARAM_LOOKBACK_DELAY_SEED) {
        if (value < 0) return LRS_E_INVAL;
        ctx->lookback_delay_seed = static_cast<unsigned int>(value);
        return LRS_OK;
    }
    return LRS_E_INVAL;
}

LRS_API lrs_status lrs_context_check(LrsContext* ctx) {
    if (!ctx) return LRS_E_INVAL;
    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return LRS_E_DEVICE;
    if (hipDeviceSynchronize() != hipSuccess) return LRS_E_DEVICE;
    unsigned int flag = 0;
    if (hipMemcpy(&flag, ctx->fixed + 1, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess)
        return LRS_E_DEVICE;
    if (flag) {
        const unsigned int zero = 0;
        (void)hipMemcpy(ctx->fixed + 1, &zero, sizeof(zero), hipMemcpyHostToDevice);
        return LRS_E_DEVICE;
    }
    return LRS_OK;
}

// ---------------------------------------------------------------------------
// scans
// ---------------------------------------------------------------------------
LRS_API lrs_status lrs_scan_fma(LrsContext* ctx, const float* a, const float* b, const float* s0,
                                float* s, float* s_final, int32_t B, int32_t T, int32_t N,
                                void* stream) {
    return scan_elem(ctx, false, a, b, s0, s, s_final, B, T, N, stream);
}

LRS_API lrs_status lrs_scan_gated(LrsContext* ctx, const float* a, const float* u,
                                  const float* s0, float* s, float* s_final, int32_t B,
                                  int32_t T, int32_t N, void* stream) {
    return scan_elem(ctx, true, a, u, s0, s, s_final, B, T, N, stream);
}

LRS_API lrs_status lrs_scan_gated_noalloc(const float* a, const float* u, const float* s0, float* s,
                                          float* s_final, int32_t B, int32_t T, int32_t N, void* stream_ptr) {
    if (!a || !u || !s || !s_final) return LRS_E_INVAL;
    int64_t seq = 0;
    if (!elem_dims_ok(B, T, N, seq)) return LRS_E_INVAL;
    if (!aligned(a, 4) || !aligned(u, 4) || !aligned(s0, 4) || !aligned(s, 4) || !aligned(s_final, 4))
        return LRS_E_INVAL;
    const size_t seq_bytes = static_cast<size_t>(seq) * sizeof(float);
    const size_t st_bytes = static_cast<size_t>(B) * N * sizeof(float);
    const Span ins[] = {{a, seq_bytes}, {u, seq_bytes}, {s0, st_bytes}};
    const Span outs[] = {{s, seq_bytes}, {s_final, st_bytes}};
    if (!outputs_disjoint(outs, 2, ins, 3)) return LRS_E_INVAL;
    // the size limit is a property of the shape alone, checked before any HIP call
    const bool al16 = aligned(a, 16) && aligned(u, 16) && aligned(s, 16);
    const lrs::ElemPlan lb = lrs::elem_plan(B, T, N, al16, lrs::kElemLookback);
    const bool multi_chunk = lb.chunks > 1;
    if (multi_chunk && lb.words > lrs::noalloc_words_capacity()) return LRS_E_UNSUPPORTED;

    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) {
        (void)hipGetLastError();
        return LRS_E_DEVICE;
    }
    // the automatic schedule's choice; under graph capture the stream schedule
    // (no scratch, and no host-side epoch or counter base for a replay to reuse)
    const int ksched = multi_chunk && !capturing(stream) &&
                               lrs::elem_auto_schedule(B, T, N, al16, device_cus(device)) == lrs::kElemLookback
                           ? lrs::kElemLookback : lrs::kElemStream;
    const lrs::ElemPlan plan = ksched == lrs::kElemLookback ? lb : lrs::elem_plan(B, T, N, al16, ksched);
    if (plan.grid > 0x7fffffff) return LRS_E_UNSUPPORTED;
    lrs::ElemParams p{};
    p.a = a;
    p.x = u;
    p.s0 = s0;
    p.s = s;
    p.s_final = s_final;
    p.B = B;
    p.T = T;
    p.N = N;
    p.gated = true;
    p.schedule = ksched;
    const int rc = lrs::launch_scan_elem_noalloc(p, plan, device, stream);
    if (rc == lrs::kNoallocUnsupported) return LRS_E_UNSUPPORTED;
    return rc == lrs::kNoallocOk ? LRS_OK : LRS_E_DEVICE;
}

LRS_API lrs_status lrs_scan_fma_backward(LrsContext* ctx, const float* a, const float* s0,
                                         const float* s, const float* ds, const float* ds_final,
                                         float* da, float* db, float* ds0, int32_t B, int32_t T,
                                         int32_t N, void* stream) {
    return scan_elem_bwd(ctx, false, a, nullptr, s0, s, ds, ds_final, da, db, ds0, B, T, N, stream);
}

LRS_API lrs_status lrs_scan_gated_backward(LrsContext* ctx, const float* a, const float* u,
                                           const float* s0, const float* s, const float* ds,
                                           const float* ds_final, float* da, float* du, float* ds0,
                                           int32_t B, int32_t T, int32_t N, void* stream) {
    return scan_elem_bwd(ctx, true, a, u, s0, s, ds, ds_final, da, du, ds0, B, T, N, stream);
}

LRS_API lrs_status lrs_step_fma(LrsContext* ctx, const float* a, const float* b, float* s,
                                int32_t B, int32_t N, void* stream) {
    return step_elem(ctx, false, a, b, s, B, N, stream);
}

LRS_API lrs_status lrs_step_gated(LrsContext* ctx, const float* a, const float* u, float* s,
                                  int32_t B, int32_t N, void* stream) {
    return step_elem(ctx, true, a, u, s, B, N, stream);
}

namespace {

// Grows a context-owned device buffer to `need` bytes.  The old buffer is
// released only after the device has finished all earlier work (see
// grow_words).  Under graph capture nothing may allocate or wait: growth is
// refused there (the caller enqueues nothing and returns the status).  Once a
// call of this context has been captured, a graph may still hold the old
// buffer, so it is retired instead of freed (lrs_context_destroy frees it).
lrs_status grow_workspace(LrsContext* ctx, void*& ptr, size_t& cap, size_t need, hipStream_t stream) {
    if (need <= cap) return LRS_OK;
    if (capturing(stream)) return LRS_E_UNSUPPORTED;
    if (ptr) {
        if (ctx->captured) {
            ctx->retired.push_back(ptr);
        } else {
            if (hipDeviceSynchronize() != hipSuccess) return LRS_E_DEVICE;
            (void)hipFree(ptr);
        }
        ptr = nullptr;
        cap = 0;
    }
    void* fresh = nullptr;
    if (hipMalloc(&fresh, need) != hipSuccess) {
        (void)hipGetLastError();
        return LRS_E_NOMEM;
    }
    ptr = fresh;
    cap = need;
    return LRS_OK;
}

}  // namespace

namespace {

// Output epilogue of a diag-outer call (all zero: none, fp32 output).
struct DiagEpilogue {
    int32_t kind = LRS_EPILOGUE_NONE;
    int32_t out_dtype = LRS_DTYPE_F32;
    const float* d_skip = nullptr;
    const lrs_bf16* gate = nullptr;
    const float* norm_weight = nullptr;
    float eps = 0.0f;
};

// Shared by the per-head (or absent) kappa, per-key kappa and epilogue calls.
lrs_status scan_diag_outer_impl(LrsContext* ctx, const lrs_bf16* q, const lrs_bf16* k, const lrs_bf16* v,
                                const float* g, int32_t decay_mode, const float* k_scale, bool kscale_key,
                                float scale, const float* s0, void* o, float* s_final, int32_t B,
                                int32_t T, int32_t H, int32_t Hg, int32_t K, int32_t V, void* stream,
                                const DiagEpilogue& epi = DiagEpilogue()) {
    if (!ctx || !q || !k || !v || !g || !o || !s_final) return LRS_E_INVAL;
    if (kscale_key && (!k_scale || decay_mode != 1)) return LRS_E_INVAL;
    if (epi.kind != LRS_EPILOGUE_NONE && epi.kind != LRS_EPILOGUE_SKIP && epi.kind != LRS_EPILOGUE_NORM_GATE)
        return LRS_E_INVAL;
    if (epi.out_dtype != LRS_DTYPE_F32 && epi.out_dtype != LRS_DTYPE_BF16) return LRS_E_INVAL;
    if ((epi.kind == LRS_EPILOGUE_SKIP && !epi.d_skip) || (epi.kind == LRS_EPILOGUE_NORM_GATE && !epi.gate))
        return LRS_E_INVAL;
    if (!(epi.eps >= 0.0f)) return LRS_E_INVAL;
    // the norm needs a whole value row in one workgroup: at most 128 columns
    if (epi.kind == LRS_EPILOGUE_NORM_GATE && V > 128) return LRS_E_UNSUPPORTED;
    const bool use_epi = epi.kind != LRS_EPILOGUE_NONE || epi.out_dtype != LRS_DTYPE_F32;
    if (use_epi && kscale_key) return LRS_E_UNSUPPORTED;
    const size_t osz = epi.out_dtype == LRS_DTYPE_BF16 ? 2 : 4;
    if (B < 1 || T < 1 || H < 1 || Hg < 1 || K < 1 || V < 1) return LRS_E_INVAL;
    if (H % Hg != 0 || (decay_mode != 0 && decay_mode != 1)) return LRS_E_INVAL;
    if (K > 128) return LRS_E_UNSUPPORTED;
    if (!aligned(q, 2) || !aligned(k, 2) || !aligned(v, 2) || !aligned(g, 4) || !aligned(k_scale, 4) ||
        !aligned(s0, 4) || !aligned(o, osz) || !aligned(s_final, 4) || !aligned(epi.d_skip, 4) ||
        !aligned(epi.gate, 2) || !aligned(epi.norm_weight, 4))
        return LRS_E_INVAL;
    int64_t bt = B;
    if (!mul_ok(bt, T)) return LRS_E_INVAL;
    int64_t nqk = bt, nv = bt, ng = bt, nst = B;
    if (!mul_ok(nqk, Hg) || !mul_ok(nqk, K) || !mul_ok(nv, H) || !mul_ok(nv, V) || !mul_ok(ng, H) ||
        (decay_mode == 1 && !mul_ok(ng, K)) || !mul_ok(nst, H) || !mul_ok(nst, K) || !mul_ok(nst, V))
        return LRS_E_INVAL;
    const size_t bqk = static_cast<size_t>(nqk) * 2, bv = static_cast<size_t>(nv) * 2;
    const size_t bg = static_cast<size_t>(ng) * 4;
    const size_t bks = static_cast<size_t>(bt) * H * (kscale_key ? K : 1) * 4;
    const size_t bo = static_cast<size_t>(nv) * osz, bst = static_cast<size_t>(nst) * 4;
    const Span ins[] = {{q, bqk}, {k, bqk}, {v, bv}, {g, bg}, {k_scale, bks}, {s0, bst},
                        {epi.d_skip, static_cast<size_t>(H) * 4}, {epi.gate, bv},
                        {epi.norm_weight, static_cast<size_t>(V) * 4}};
    const Span outs[] = {{o, bo}, {s_final, bst}};
    if (!outputs_disjoint(outs, 2, ins, 9)) return LRS_E_INVAL;

    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return LRS_E_DEVICE;
    lrs::DiagParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.decay_mode = decay_mode;
    p.k_scale = k_scale;
    p.k_scale_key = kscale_key ? 1 : 0;
    p.scale = scale;
    p.s0 = s0;
    p.o = static_cast<float*>(o);
    p.s_final = s_final;
    p.epi_kind = epi.kind;
    p.out_bf16 = epi.out_dtype == LRS_DTYPE_BF16 ? 1 : 0;
    p.d_skip = epi.kind == LRS_EPILOGUE_SKIP ? epi.d_skip : nullptr;
    p.gate = epi.kind == LRS_EPILOGUE_NORM_GATE ? epi.gate : nullptr;
    p.norm_w = epi.kind == LRS_EPILOGUE_NORM_GATE ? epi.norm_weight : nullptr;
    p.eps = epi.eps;
    p.B = B;
    p.T = T;
    p.H = H;
    p.Hg = Hg;
    p.K = K;
    p.V = V;
    // the vector path addresses one batch row of each tensor with 32-bit buffer offsets
    const int64_t row_bytes = (static_cast<int64_t>(T) + 64) * H * (K > V ? K : V) * 4;
    p.vec = (K % 8 == 0 && V % 8 == 0 && aligned(q, 16) && aligned(k, 16) && aligned(v, 16) &&
             aligned(g, 16) && aligned(o, 16) && (!kscale_key || aligned(k_scale, 16)) &&
             (!epi.gate || aligned(epi.gate, 16)) && row_bytes < (int64_t{1} << 31)) ? 1 : 0;
    const lrs::DiagPlan plan = lrs::diag_outer_plan(B, T, H, V, K, decay_mode, kscale_key, p.vec != 0,
                                                    ctx->num_cus, ctx->diag_segments);
    const int64_t grid = static_cast<int64_t>(B) * H * plan.vtiles * plan.nseg;
    // (the prefix over segments launches up to 16 workgroups per (batch, head, V-tile))
    if (grid > 0x7fffffff || static_cast<int64_t>(B) * H * plan.vtiles * 16 > 0x7fffffff) return LRS_E_UNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const lrs_status ws = grow_workspace(ctx, ctx->diag_ws, ctx->diag_ws_bytes,
                                         lrs::diag_outer_workspace_bytes(B, H, K, V, plan.nseg), st);
    if (ws != LRS_OK) return ws;
    if (lrs::launch_scan_diag_outer(p, plan, ctx->diag_ws, st) != hipSuccess) return LRS_E_DEVICE;
    if (capturing(st)) ctx->captured = true;
    ctx->last_stream = st;
    ctx->used = true;
    return LRS_OK;
}

}  // namespace

LRS_API lrs_status lrs_scan_diag_outer(LrsContext* ctx, const lrs_bf16* q, const lrs_bf16* k,
                                       const lrs_bf16* v, const float* g, int32_t decay_mode,
                                       const float* k_scale, float scale, const float* s0,
                                       float* o, float* s_final, int32_t B, int32_t T, int32_t H,
                                       int32_t Hg, int32_t K, int32_t V, void* stream) {
    return scan_diag_outer_impl(ctx, q, k, v, g, decay_mode, k_scale, false, scale, s0, o, s_final, B, T, H,
                                Hg, K, V, stream);
}

LRS_API lrs_status lrs_scan_diag_outer_epilogue(LrsContext* ctx, const lrs_bf16* q, const lrs_bf16* k,
                                                const lrs_bf16* v, const float* g, int32_t decay_mode,
                                                const float* k_scale, float scale, const float* s0,
                                                int32_t epilogue, const float* d_skip, const lrs_bf16* gate,
                                                const float* norm_weight, float eps, int32_t out_dtype, void* o,
                                                float* s_final, int32_t B, int32_t T, int32_t H, int32_t Hg,
                                                int32_t K, int32_t V, void* stream) {
    DiagEpilogue epi;
    epi.kind = epilogue;
    epi.out_dtype = out_dtype;
    epi.d_skip = d_skip;
    epi.gate = gate;
    epi.norm_weight = norm_weight;
    epi.eps = eps;
    return scan_diag_outer_impl(ctx, q, k, v, g, decay_mode, k_scale, false, scale, s0, o, s_final, B, T, H, Hg,
                                K, V, stream, epi);
}

LRS_API lrs_status lrs_scan_diag_outer_keyscale(LrsContext* ctx, const lrs_bf16* q, const lrs_bf16* k,
                                                const lrs_bf16* v, const float* g, const float* k_scale,
                                                float scale, const float* s0, float* o, float* s_final,
                                                int32_t B, int32_t T, int32_t H, int32_t Hg, int32_t K,
                                                int32_t V, void* stream) {
    return scan_diag_outer_impl(ctx, q, k, v, g, 1, k_scale, true, scale, s0, o, s_final, B, T, H, Hg, K, V,
                                stream);
}

namespace {

// Shared by the plain and decayed delta-rule calls (g == NULL: plain), with an
// fp32 or bf16 output.
lrs_status scan_delta_impl(LrsContext* ctx, const lrs_bf16* q, const lrs_bf16* k, const lrs_bf16* v,
                           const float* g, const float* beta, float scale, const float* s0, void* o,
                           float* s_final, int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                           void* stream, int32_t out_dtype = LRS_DTYPE_F32) {
    const bool decay = g != nullptr;
    if (!ctx || !q || !k || !v || !beta || !o || !s_final) return LRS_E_INVAL;
    if (out_dtype != LRS_DTYPE_F32 && out_dtype != LRS_DTYPE_BF16) return LRS_E_INVAL;
    const size_t osz = out_dtype == LRS_DTYPE_BF16 ? 2 : 4;
    if (B < 1 || T < 1 || H < 1 || K < 1 || V < 1) return LRS_E_INVAL;
    if (K > (decay ? lrs::delta_decay_max_k() : 128)) return LRS_E_UNSUPPORTED;
    if (!aligned(q, 2) || !aligned(k, 2) || !aligned(v, 2) || !aligned(g, 4) || !aligned(beta, 4) ||
        !aligned(s0, 4) || !aligned(o, osz) || !aligned(s_final, 4))
        return LRS_E_INVAL;
    int64_t bth = B;
    if (!mul_ok(bth, T) || !mul_ok(bth, H)) return LRS_E_INVAL;
    int64_t nqk = bth, nv = bth, nst = B;
    if (!mul_ok(nqk, K) || !mul_ok(nv, V) || !mul_ok(nst, H) || !mul_ok(nst, K) || !mul_ok(nst, V))
        return LRS_E_INVAL;
    const size_t bqk = static_cast<size_t>(nqk) * 2, bv = static_cast<size_t>(nv) * 2;
    const size_t bb = static_cast<size_t>(bth) * 4, bo = static_cast<size_t>(nv) * osz;
    const size_t bst = static_cast<size_t>(nst) * 4, bg = decay ? static_cast<size_t>(nqk) * 4 : 0;
    const Span ins[] = {{q, bqk}, {k, bqk}, {v, bv}, {beta, bb}, {s0, bst}, {g, bg}};
    const Span outs[] = {{o, bo}, {s_final, bst}};
    if (!outputs_disjoint(outs, 2, ins, 6)) return LRS_E_INVAL;

    const int64_t nchunks = (static_cast<int64_t>(T) + 63) / 64;
    const int64_t vtiles = (V + lrs::delta_vtile() - 1) / lrs::delta_vtile();
    if (static_cast<int64_t>(B) * H * nchunks > 0x7fffffff || static_cast<int64_t>(B) * H * vtiles > 0x7fffffff)
        return LRS_E_UNSUPPORTED;
    // the scan kernel addresses one (batch, head) slice of the workspace with 32-bit offsets
    if (lrs::delta_chunk_workspace_bytes(1, T, 1, K, decay) >= (size_t{1} << 31)) return LRS_E_UNSUPPORTED;
    const int nseg = lrs::delta_plan_segments(B, T, H, K, V, ctx->num_cus, ctx->delta_segments);

    hipStream_t st = static_cast<hipStream_t>(stream);
    DeviceGuard guard(ctx->device);
    if (!guard.ok()) return LRS_E_DEVICE;
    const lrs_status ws = grow_workspace(ctx, ctx->delta_ws, ctx->delta_ws_bytes,
                                         lrs::delta_workspace_bytes(B, T, H, K, V, decay, nseg), st);
    if (ws != LRS_OK) return ws;
    lrs::DeltaParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.scale = scale;
    p.s0 = s0;
    p.o = static_cast<float*>(o);
    p.s_final = s_final;
    p.B = B;
    p.T = T;
    p.H = H;
    p.K = K;
    p.V = V;
    p.out_bf16 = out_dtype == LRS_DTYPE_BF16 ? 1 : 0;
    p.nseg = nseg;
    // the vector path addresses one batch row of each tensor with 32-bit buffer
    // offsets, and stores each lane's four outputs at once (16 or 8 bytes)
    const int64_t row_bytes = (static_cast<int64_t>(T) + 64) * H * (K > V ? K : V) * 4;
    p.vec = (K % 8 == 0 && V % 8 == 0 && aligned(q, 16) && aligned(k, 16) && aligned(v, 16) &&
             aligned(g, 16) && aligned(o, 16) && row_bytes < (int64_t{1} << 31)) ? 1 : 0;
    if (lrs::launch_scan_delta(p, ctx->delta_ws, st) != hipSuccess) return LRS_E_DEVICE;
    if (capturing(st)) ctx->captured = true;
    ctx->last_stream = st;
    ctx->used = true;
    return LRS_OK;
}

}  // namespace

LRS_API lrs_status lrs_scan_delta(LrsContext* ctx, const lrs_bf16* q, const lrs_bf16* k,
                                  const lrs_bf16* v, const float* beta, float scale,
                                  const float* s0, float* o, float* s_final, int32_t B, int32_t T,
                                  int32_t H, int32_t K, int32_t V, void* stream) {
    return scan_delta_impl(ctx, q, k, v, nullptr, beta, scale, s0, o, s_final, B, T, H, K, V, stream);
}

LRS_API lrs_status lrs_scan_delta_decay(LrsContext* ctx, const lrs_bf16* q, const lrs_bf16* k,
                                        const lrs_bf16* v, const float* g, const float* beta,
                                        float scale, const float* s0, float* o, float* s_final,
                                        int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                        void* stream) {
    if (!g) return LRS_E_INVAL;
    return scan_delta_impl(ctx, q, k, v, g, beta, scale, s0, o, s_final, B, T, H, K, V, stream);
}

LRS_API lrs_status lrs_scan_delta_out(LrsContext* ctx, const lrs_bf16* q, const lrs_bf16* k, const lrs_bf16* v,
                                      const float* g, const float* beta, float scale, const float* s0,
                                      int32_t out_dtype, void* o, float* s_final, int32_t B, int32_t T, int32_t H,
                                      int32_t K, int32_t V, void* stream) {
    return scan_delta_impl(ctx, q, k, v, g, beta, scale, s0, o, s_final, B, T, H, K, V, stream, out_dtype);
}
