// bf16 matrix-core helpers for the chunked prefill kernels (gfx950): bf16
// packing and hi / lo splitting, k32 operand fragments from LDS, and the
// bounded LDS counters that let the waves of one workgroup hand work to each
// other without workgroup-wide barriers.
#pragma once

#include "kda_common.hpp"

namespace kda {
namespace b16 {

__device__ __forceinline__ void signal(unsigned* c, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane == 0) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Waits until *c >= target.  The wait is bounded by spin_limit polls: a wait
// that runs out sets the workgroup's abort word, after which every wait
// returns at once, so the kernel always ends (with meaningless results in that
// case, which the kernel reports to the host through its WaitCtl).  All waves
// of a workgroup are resident together, so the default bound is never reached
// in practice.
__device__ __forceinline__ void wait_for(unsigned* c, unsigned target, unsigned* abort_word,
                                         unsigned spin_limit) {
    unsigned spins = 0;
    while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target) {
        if (__hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0u)
            break;
        __builtin_amdgcn_s_sleep(1);
        if (++spins >= spin_limit) {
            __hip_atomic_store(abort_word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            break;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// k32 A-operand fragment of row `row` of a row-major bf16 matrix in LDS:
// values 0..3 carry k = k0 + 4g + e, values 4..7 carry k = k0 + 16 + 4g + e.
__device__ __forceinline__ bf16x8 frag_row(const uint16_t* base, int pitch, int row, int k0,
                                           int gq) {
    const uint16_t* p = base + row * pitch + k0 + 4 * gq;
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    const uint2 b = *reinterpret_cast<const uint2*>(p + 16);
    const uint4 u = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, u);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to a pair of bf16 (round to nearest even) in one register.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Eight floats to a bf16x8 operand, in order.
__device__ __forceinline__ bf16x8 pack8(const float* x) {
    const u32x4 u = {pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
    return __builtin_bit_cast(bf16x8, u);
}

// The k order of the products for a B operand held in accumulator tiles lo
// (k0..k0+15) and hi (k0+16..k0+31).
__device__ __forceinline__ bf16x8 pack_b(f32x4 lo, f32x4 hi) {
    const u32x4 u = {pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]), pack2(hi[2], hi[3])};
    return __builtin_bit_cast(bf16x8, u);
}

// hi = bf16(x), lo = bf16(x - hi): x as a bf16 hi + lo pair (about 16 bits).
__device__ __forceinline__ void split_b(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
    hi = pack_b(a, b);
    const u32x4 h = __builtin_bit_cast(u32x4, hi);
    f32x4 ra, rb;
    ra[0] = __builtin_bit_cast(float, h[0] << 16);
    ra[1] = __builtin_bit_cast(float, h[0] & 0xffff0000u);
    ra[2] = __builtin_bit_cast(float, h[1] << 16);
    ra[3] = __builtin_bit_cast(float, h[1] & 0xffff0000u);
    rb[0] = __builtin_bit_cast(float, h[2] << 16);
    rb[1] = __builtin_bit_cast(float, h[2] & 0xffff0000u);
    rb[2] = __builtin_bit_cast(float, h[3] << 16);
    rb[3] = __builtin_bit_cast(float, h[3] & 0xffff0000u);
    lo = pack_b(a - ra, b - rb);
}

// The same split for four consecutive values, as two 8-byte rows (hi, lo).
__device__ __forceinline__ void split4(const float* x, uint2& hi, uint2& lo) {
    hi = uint2{pack2(x[0], x[1]), pack2(x[2], x[3])};
    const float r0 = __builtin_bit_cast(float, hi.x << 16), r1 = __builtin_bit_cast(float, hi.x & 0xffff0000u);
    const float r2 = __builtin_bit_cast(float, hi.y << 16), r3 = __builtin_bit_cast(float, hi.y & 0xffff0000u);
    lo = uint2{pack2(x[0] - r0, x[1] - r1), pack2(x[2] - r2, x[3] - r3)};
}

__device__ __forceinline__ f32x4 mma(f32x4 acc, bf16x8 a, bf16x8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// ---- k32 operand fragments held as bf16 hi / lo pairs in LDS -----------------
// A fragment is 16 rows x 32 k: 1 KB of hi and 1 KB of lo, lane (n, g) of the
// reading wave at u32x4 entry n + 16 g, holding row n with k = k0 + 4g + e
// (values 0..3) and k0 + 16 + 4g + e (values 4..7).
constexpr int kFragLanes = 64;  // u32x4 entries of one fragment

// Four values along k of fragment f at lane slot (n, g), half h (values 0..3
// or 4..7): written as bf16 hi and lo into the two fragment arrays.
__device__ __forceinline__ void put_frag_hl(u32x4* hi, u32x4* lo, int f, int n, int g, int h,
                                            float4 x) {
    const float a[4] = {x.x, x.y, x.z, x.w};
    uint2 vh, vl;
    split4(a, vh, vl);
    reinterpret_cast<uint2*>(&hi[kFragLanes * f + n + 16 * g])[h] = vh;
    reinterpret_cast<uint2*>(&lo[kFragLanes * f + n + 16 * g])[h] = vl;
}
__device__ __forceinline__ bf16x8 frag_at(const u32x4* base, int f, int lane) {
    return __builtin_bit_cast(bf16x8, base[kFragLanes * f + lane]);
}
// acc += A B with both factors as hi / lo pairs (lo hi + hi lo + hi hi)
__device__ __forceinline__ f32x4 mma3(f32x4 acc, bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl) {
    acc = mma(acc, al, bh);
    acc = mma(acc, ah, bl);
    return mma(acc, ah, bh);
}
// The six nonzero k32 fragments of a lower-triangular [64][64] matrix (row
// tile rt, k32 block s2): (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
__host__ __device__ constexpr int tri_rt(int f) { return f < 2 ? f : 2 + ((f - 2) >> 1); }
__host__ __device__ constexpr int tri_s2(int f) { return f < 2 ? 0 : (f - 2) & 1; }

}  // namespace b16
}  // namespace kda
