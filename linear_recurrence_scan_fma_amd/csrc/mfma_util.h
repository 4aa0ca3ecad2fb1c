// Small helpers for the matrix-state scans: bf16 conversion and splitting,
// MFMA fragment loads from LDS, and the 16x16x32 bf16 matrix-core op.
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (64 lanes, g = lane / 16):
//   A fragment: row (lane % 16), k = 8g .. 8g+7           (8 bf16 per lane)
//   B fragment: col (lane % 16), k = 8g .. 8g+7
//   D fragment: col (lane % 16), rows 4g .. 4g+3           (4 fp32 per lane)
// Every operand is kept in LDS as a row-major array whose rows are the M (or N)
// index and whose columns are the contraction index, so both A and B fragments
// are one aligned 16-byte LDS read per lane.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace lrs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u16 f2bf(float x) {
    __bf16 b = static_cast<__bf16>(x);  // round to nearest even
    return __builtin_bit_cast(u16, b);
}

__device__ __forceinline__ float bf2f(u16 h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi): about 16 significant bits.
__device__ __forceinline__ void split_bf16(float x, u16& hi, u16& lo) {
    hi = f2bf(x);
    lo = f2bf(x - bf2f(hi));
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two values at once: hi and lo come back as packed bf16 pairs (the first
// value in the low half), with a + b ~= hi + lo as in split_bf16.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    const float ha = __uint_as_float(h << 16), hb = __uint_as_float(h & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a - ha, b - hb}, bf16x2));
    hi = h;
}

// Eight values (two groups of four) as hi and lo bf16x8 operands.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split2(x[2 * i], x[2 * i + 1], h[i], l[i]);
    hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}

template <int LD>
__device__ __forceinline__ bf16x8 frag(const u16* base, int r0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8*>(base + (r0 + (lane & 15)) * LD + k0 + 8 * (lane >> 4));
}

// The same fragment from an array whose rows are only 8-byte aligned: two
// 8-byte LDS reads per lane.
template <int LD>
__device__ __forceinline__ bf16x8 frag_b64(const u16* base, int r0, int k0, int lane) {
    const u16* p = base + (r0 + (lane & 15)) * LD + k0 + 8 * (lane >> 4);
    const u32x2 a = *reinterpret_cast<const u32x2*>(p);
    const u32x2 b = *reinterpret_cast<const u32x2*>(p + 4);
    return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
}

// The contraction index of a 16x16x32 product may be permuted as long as both
// operands agree.  "Slot" operands give lane group g the contraction indices
// {k0 + 4g .. k0 + 4g + 3} u {k0 + 16 + 4g .. k0 + 16 + 4g + 3}: exactly what
// two 16x16 accumulator tiles hold in rows 4g .. 4g + 3, so accumulators can
// feed the next product without leaving their registers.

// Slot operand from a row-major array: row `rowp` at column k0 + 4g (the
// caller adds k0 + 4g), two 8-byte LDS reads.
__device__ __forceinline__ bf16x8 slot_frag(const u16* rowp) {
    const u32x2 a = *reinterpret_cast<const u32x2*>(rowp);
    const u32x2 b = *reinterpret_cast<const u32x2*>(rowp + 16);
    return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
}

// Transposed slot operand from a row-major [k][n] bf16 array in LDS: lane j of
// 16-lane group g receives M[k0 .. k0+3][n0 + j] and M[k0+16 .. k0+19][n0 + j]
// with k0 = kb + 4g (ds_read_b64_tr_b16: lane i of a group supplies row
// k0 + i/4, columns n0 + 4(i%4)).
template <int LD>
__device__ __forceinline__ bf16x8 tr_frag(const u16* m, int kb, int n0, int lane) {
    const int i16 = lane & 15, k0 = kb + 4 * (lane >> 4);
    const u16* pa = m + (k0 + (i16 >> 2)) * LD + n0 + 4 * (i16 & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa + 16 * LD));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() {
    f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    return z;
}

// 8 consecutive bf16 (16 bytes) of a row of length n starting at column c0;
// zero beyond n.  `vec` says the row start is 16-byte aligned and n % 8 == 0.
__device__ __forceinline__ u32x4 load8_bf16(const u16* row, int c0, int n, bool vec) {
    if (vec) {
        // zero first, then the guarded load: a zero written after a masked load
        // to the same registers would force the load to drain first
        u32x4 r = {0u, 0u, 0u, 0u};
        if (c0 + 8 <= n) r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + c0));
        return r;
    }
    u16 t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = (c0 + e < n) ? row[c0 + e] : static_cast<u16>(0);
    return u32x4{t[0] | (static_cast<uint32_t>(t[1]) << 16), t[2] | (static_cast<uint32_t>(t[3]) << 16),
                 t[4] | (static_cast<uint32_t>(t[5]) << 16), t[6] | (static_cast<uint32_t>(t[7]) << 16)};
}

__device__ __forceinline__ u16 piece_elem(const u32x4& v, int e) {
    const uint32_t w = e < 2 ? v.x : (e < 4 ? v.y : (e < 6 ? v.z : v.w));
    return static_cast<u16>((e & 1) ? (w >> 16) : (w & 0xffff));
}

// Raw buffer access.  A buffer resource covers [base, base + bytes); a load
// whose offset falls outside returns zero without touching memory.  The kernels
// give each (batch) row of a tensor its own resource, so time steps past T and
// columns past K or V read as zero with no branch, and the prefetch of the next
// chunk stays a straight run of loads.
typedef __amdgpu_buffer_rsrc_t BufRes;
constexpr int kBufOOB = 0x7fffffff;   // an offset past every resource

__device__ __forceinline__ BufRes make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(BufRes r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ float buf_load_f32(BufRes r, int off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// A resource over [base + skip, base + bytes): a loop over time steps moves its
// window with scalar arithmetic only, keeping per-lane offsets loop-invariant.
// The range check of a raw buffer access covers the per-lane offset (plus the
// instruction's immediate), so accesses past the window read zero or are
// dropped.
__device__ __forceinline__ BufRes make_rsrc_window(const void* base, int64_t bytes, int64_t skip) {
    const int64_t left = bytes > skip ? bytes - skip : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(base)) + skip,
                                             static_cast<short>(0), static_cast<int>(left), 0x00020000);
}

__device__ __forceinline__ void buf_store16(u32x4 x, BufRes r, int off) {
    __builtin_amdgcn_raw_buffer_store_b128(x, r, off, 0, 0);
}

// XCD-aware workgroup order: the hardware hands consecutive workgroup ids to
// the 8 XCDs in turn; remap so that consecutive logical ids share an XCD
// (and its L2) when the grid divides evenly.
__device__ __forceinline__ int xcd_logical_id(int bid, int grid) {
    if (grid % 8 != 0) return bid;
    return (bid % 8) * (grid / 8) + bid / 8;
}

}  // namespace lrs
