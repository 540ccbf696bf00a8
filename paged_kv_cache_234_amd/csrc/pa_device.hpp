// Device-side building blocks for the paged-attention kernels (gfx950 only).
//
// Everything here is CDNA4-specific: 64-lane wavefronts, the gfx950 MFMA
// shapes v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x4_f32, the OCP fp8
// conversion instructions and 16-byte global loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 16;                 // tokens per KV block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum CacheKind { kF32 = 0, kBF16 = 1, kFP8 = 2 };

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---- MFMA wrappers ---------------------------------------------------------
// 16x16x32 bf16: lane l supplies A[row l%16][k 8*(l/16) .. +7] and
// B[k 8*(l/16) .. +7][col l%16]; C/D lane l holds rows 4*(l/16)+i, col l%16.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x4 fp32: lane l supplies A[row l%16][k l/16] and B[k l/16][col l%16].
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---- conversions -----------------------------------------------------------
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 OCP e4m3 codes (two dwords) -> 8 bf16 (exact: every e4m3 value is a bf16).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// ---- cross-lane reductions over the four 16-lane groups --------------------
// gfx950's v_permlane32_swap / v_permlane16_swap exchange 32- and 16-lane
// halves between two VGPRs without going through LDS: starting from two
// copies of x, lane l ends up holding x[l] and x[l^32] (x[l^16]) across the
// two registers, so max/sum over lanes {l, l^16, l^32, l^48} is four VALU ops.
// The swaps are issued through inline asm on two distinct register operands:
// the compiler's builtin folds a swap of two equal inputs to two equal
// outputs, which drops the exchange.  The s_nop covers the VALU-write ->
// permlane-read hazard.
__device__ __forceinline__ void permlane32_swap(uint32_t& a, uint32_t& b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane16_swap(uint32_t& a, uint32_t& b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_over_groups(float x) {
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    permlane32_swap(a, b);
    uint32_t c = __builtin_bit_cast(uint32_t,
                                    fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)));
    uint32_t d = c;
    permlane16_swap(c, d);
    return fmaxf(__builtin_bit_cast(float, c), __builtin_bit_cast(float, d));
}
// The same maximum, NaN-propagating (v_maximum3): unlike fmaxf it needs no
// canonicalisation of the exchanged values.
__device__ __forceinline__ float fmax_nan(float a, float b) {
    return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float max_over_groups_nan(float x) {
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    permlane32_swap(a, b);
    uint32_t c = __builtin_bit_cast(uint32_t,
                                    fmax_nan(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)));
    uint32_t d = c;
    permlane16_swap(c, d);
    return fmax_nan(__builtin_bit_cast(float, c), __builtin_bit_cast(float, d));
}
__device__ __forceinline__ float sum_over_groups(float x) {
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    permlane32_swap(a, b);
    uint32_t c = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
    uint32_t d = c;
    permlane16_swap(c, d);
    return __builtin_bit_cast(float, c) + __builtin_bit_cast(float, d);
}

// Load through the constant address space: for memory the kernel never
// writes (block tables, scales, group lists).  A wave-uniform address then
// becomes a scalar load, whose completion is tracked apart from the K/V
// vector loads still in flight.
template <class T> __device__ __forceinline__ T load_invariant(const T* p) {
    return *(const __attribute__((address_space(4))) T*)(p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- 16-byte global loads (non-temporal for streamed KV) --------------------
__device__ __forceinline__ u32x4 load16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 load16_cached(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// ---- workgroup -> work-item mapping that keeps neighbours on one XCD --------
// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2.  Renumber them so that every run of 8 consecutive work items executes
// on one XCD at about the same time, while successive runs rotate over the
// XCDs: items that read the same KV blocks (the sequences of a
// prefix-sharing group, laid out next to each other) share an L2, and the
// work still spreads evenly over the chip at 8-item granularity.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    constexpr int kXcd = 8, kRun = 8, kRound = kXcd * kRun;
    if (bid >= (nblocks / kRound) * kRound) return bid;     // incomplete last round
    const int slot = bid / kXcd, xcd = bid % kXcd;
    return kRound * (slot / kRun) + kRun * xcd + slot % kRun;
}

}  // namespace pa
