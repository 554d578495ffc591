// Device-side building blocks shared by the libkda kernels (gfx950 only):
// element types, bf16 packing, matrix-core (MFMA) fragment helpers, the
// 16-lane prefix scan used for in-chunk decay sums, and lane bookkeeping.
//
// MFMA register layouts used throughout (64-lane wavefront, g = lane / 16,
// n = lane % 16):
//   16x16 accumulator (any 16x16 MFMA): lane holds C[4g + e][n], e = 0..3.
//   k32 step (v_mfma_f32_16x16x32_bf16): lane holds 8 operand values; for the
//     A operand they belong to row n, for the B operand to column n.  Which k
//     index each of the 8 values carries is a free choice as long as A and B
//     agree; every call site states its k order.
//   k16 step (v_mfma_f32_16x16x16_bf16): 4 values per lane at k = 4g + e.
//     The B operand of a k16 step has exactly the accumulator layout, so a
//     16x16 result can feed the next product without any data movement.
// The fp32 policy runs the same data layouts on v_mfma_f32_16x16x4_f32: one
// k32 step is 8 such MFMAs (value e of every lane forms the e-th), a k16 step
// is 4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kD = 128;     // head dimension (d_k = d_v)
constexpr int kChunk = 64;  // tokens per chunk
constexpr int kSub = 16;    // rows per sub-block of a chunk
constexpr float kNormEps = 1e-6f;
constexpr float kLog2e = 1.4426950408889634f;  // exp(x) = exp2(x log2 e)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint16_t f2bf(float x) {
    // v_cvt_pk_bf16_f32: round to nearest even, NaN preserved
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ float bf2f(uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// Inclusive prefix sum across the 16 lanes of each DPP row (lanes 16r..16r+15).
__device__ __forceinline__ float row16_inclusive_scan(float x) {
#define KDA_ROW_SHR_ADD(n)                                                           \
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(                      \
                                       0, __builtin_bit_cast(int, x), 0x110 + (n), \
                                       0xf, 0xf, true))
    KDA_ROW_SHR_ADD(1);
    KDA_ROW_SHR_ADD(2);
    KDA_ROW_SHR_ADD(4);
    KDA_ROW_SHR_ADD(8);
#undef KDA_ROW_SHR_ADD
    return x;
}

__device__ __forceinline__ float fast_exp(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// ---------------------------------------------------------------------------
// Element policies by I/O type.  Prec<false>: bf16 q / k / v / out (the
// decode step converts on load and store).  Prec<true>: fp32 I/O, and the fp32
// operands and 16x16x4 fp32 products of the fp32 chunked prefill.
// ---------------------------------------------------------------------------
template <bool F32>
struct Prec;

template <>
struct Prec<false> {  // bf16 I/O (the decode step)
    using io_t = uint16_t;
    __device__ static __forceinline__ float from_io(io_t x) { return bf2f(x); }
    __device__ static __forceinline__ io_t to_io(float x) { return f2bf(x); }
};

template <>
struct Prec<true> {
    using io_t = float;
    using st_t = float;
    struct F8 { float v[8]; };
    struct F4 { float v[4]; };

    __device__ static __forceinline__ st_t to_st(float x) { return x; }
    __device__ static __forceinline__ float from_st(st_t x) { return x; }
    __device__ static __forceinline__ float from_io(io_t x) { return x; }
    __device__ static __forceinline__ io_t to_io(float x) { return x; }

    __device__ static __forceinline__ F8 pack8(const float* x) {
        F8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f.v[e] = x[e];
        return f;
    }
    __device__ static __forceinline__ F8 pack8(f32x4 lo, f32x4 hi) {
        F8 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f.v[e] = lo[e];
            f.v[4 + e] = hi[e];
        }
        return f;
    }
    __device__ static __forceinline__ F4 pack4(f32x4 x) {
        F4 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f.v[e] = x[e];
        return f;
    }
    __device__ static __forceinline__ f32x4 mma32(f32x4 acc, const F8& a, const F8& b) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
        return acc;
    }
    __device__ static __forceinline__ f32x4 mma16(f32x4 acc, const F4& a, const F4& b) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
        return acc;
    }
};

// Load 8 consecutive io elements as fp32 (16-byte aligned bf16 / 2 x 16 B fp32).
__device__ __forceinline__ void load8(const uint16_t* p, float* x) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
        x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float* p, float* x) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

}  // namespace kda
