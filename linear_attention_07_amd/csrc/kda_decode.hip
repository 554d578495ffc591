// One-token KDA decode step (the pages' fused_recurrent_kda): Kimi-K3 深度解析
// blog, section 三 (decay the state per key channel, predict v from the
// decayed state, write beta * error along the key); 深入 Kimi-K3 thread, KDA
// paragraph (q/k L2-normalised in the kernel; the state is the whole carried
// context, the same size at any context length).
//
// The step touches every state entry exactly once.  With S' = Diag(exp g) S,
//   p = S'^T kh,  r = S'^T qh,  u = beta (v - p),
//   o = scale (r + (kh . qh) u)        since (S' + kh u^T)^T qh = r + (kh.qh) u,
//   S = S' + kh u^T,
// so one read and one write of the 64 KB fp32 state per (batch, head) suffice:
// the decode is an HBM stream (about 0.86 flop per byte).
//
// Layout: one 256-thread workgroup per (b, h).  Thread t owns value columns
// 4*(t%32) .. +3 of key rows (t/32) + 8m, m = 0..15, held in registers between
// the column reductions and the write-back; a wave's load instruction covers
// two whole 512-byte state rows.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

template <bool F32>
__global__ __launch_bounds__(256) void kda_decode_kernel(
    const typename Prec<F32>::io_t* __restrict__ q, const typename Prec<F32>::io_t* __restrict__ k,
    const typename Prec<F32>::io_t* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, float scale, float* __restrict__ S,
    typename Prec<F32>::io_t* __restrict__ out) {
    using P = Prec<F32>;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int cg = tid & 31, rg = tid >> 5;
    const int64_t bh = blockIdx.x;

    float* Sb = S + bh * (kD * kD);
    f32x4 s[16];
#pragma unroll
    for (int m = 0; m < 16; ++m)
        s[m] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(Sb + (rg + 8 * m) * kD + 4 * cg));

    __shared__ float sq[kD], sk[kD], sa[kD], sv[kD];
    __shared__ float4 red[4][2][32];
    if (tid < kD) {
        sq[tid] = P::from_io(q[bh * kD + tid]);
        sk[tid] = P::from_io(k[bh * kD + tid]);
        sa[tid] = fast_exp(g[bh * kD + tid]);
    } else {
        sv[tid - kD] = P::from_io(v[bh * kD + tid - kD]);
    }
    const float bt = beta[bh];
    __syncthreads();

    // |q|^2, |k|^2 and q.k (every wave reduces all 128 channels itself)
    float a0 = sq[lane], a1 = sq[lane + 64], b0 = sk[lane], b1 = sk[lane + 64];
    float ssq = a0 * a0 + a1 * a1, ssk = b0 * b0 + b1 * b1, sqk = a0 * b0 + a1 * b1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        ssq += __shfl_xor(ssq, off);
        ssk += __shfl_xor(ssk, off);
        sqk += __shfl_xor(sqk, off);
    }
    const float iq = 1.0f / sqrtf(ssq + kNormEps);
    const float ik = 1.0f / sqrtf(ssk + kNormEps);
    const float kq = sqk * iq * ik;

    float4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int row = rg + 8 * m;
        const float a = sa[row], kk = sk[row], qq = sq[row];
        s[m].x *= a; s[m].y *= a; s[m].z *= a; s[m].w *= a;
        p.x += kk * s[m].x; p.y += kk * s[m].y; p.z += kk * s[m].z; p.w += kk * s[m].w;
        r.x += qq * s[m].x; r.y += qq * s[m].y; r.z += qq * s[m].z; r.w += qq * s[m].w;
    }
    // lanes l and l^32 hold the same columns for adjacent row groups
    p.x += __shfl_xor(p.x, 32); p.y += __shfl_xor(p.y, 32);
    p.z += __shfl_xor(p.z, 32); p.w += __shfl_xor(p.w, 32);
    r.x += __shfl_xor(r.x, 32); r.y += __shfl_xor(r.y, 32);
    r.z += __shfl_xor(r.z, 32); r.w += __shfl_xor(r.w, 32);
    if (lane < 32) {
        red[wv][0][cg] = p;
        red[wv][1][cg] = r;
    }
    __syncthreads();
    p = red[0][0][cg]; r = red[0][1][cg];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
        const float4 pp = red[w][0][cg], rr = red[w][1][cg];
        p.x += pp.x; p.y += pp.y; p.z += pp.z; p.w += pp.w;
        r.x += rr.x; r.y += rr.y; r.z += rr.z; r.w += rr.w;
    }
    float u[4], o[4];
    const float pv[4] = {p.x, p.y, p.z, p.w}, rv[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        u[c] = bt * (sv[4 * cg + c] - pv[c] * ik);
        o[c] = scale * (rv[c] * iq + kq * u[c]);
    }
    if (rg == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) out[bh * kD + 4 * cg + c] = P::to_io(o[c]);
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const float kk = sk[rg + 8 * m] * ik;
        s[m].x += kk * u[0]; s[m].y += kk * u[1]; s[m].z += kk * u[2]; s[m].w += kk * u[3];
        __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4*>(Sb + (rg + 8 * m) * kD + 4 * cg));
    }
}

template <bool F32>
hipError_t launch_decode(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float scale, float* S, void* out, int B, int H,
                         hipStream_t stream) {
    using io = typename Prec<F32>::io_t;
    const unsigned nblk = (unsigned)((int64_t)B * H);
    hipLaunchKernelGGL(kda_decode_kernel<F32>, dim3(nblk), dim3(256), 0, stream,
                       static_cast<const io*>(q), static_cast<const io*>(k),
                       static_cast<const io*>(v), g, beta, scale, S, static_cast<io*>(out));
    return hipGetLastError();
}

template hipError_t launch_decode<false>(const void*, const void*, const void*, const float*,
                                         const float*, float, float*, void*, int, int,
                                         hipStream_t);
template hipError_t launch_decode<true>(const void*, const void*, const void*, const float*,
                                        const float*, float, float*, void*, int, int,
                                        hipStream_t);

}  // namespace kda
