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
// Layout: each wave owns half of one state, value columns 64*half .. +63 for
// all 128 key rows.  Lane (cg = lane%16, rg = lane/16) holds columns
// 64*half + 4cg .. +3 of rows 32rg .. 32rg+31 (128 fp32 in registers), so the
// reductions over key rows are a sum over the lane's 32 rows plus two lane
// shuffles: no LDS round trip and no workgroup barrier between the read and
// the write of the state.  A 256-thread workgroup serves two (b, h).
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

template <bool F32>
__global__ __launch_bounds__(256) void kda_decode_kernel(
    const typename Prec<F32>::io_t* __restrict__ q, const typename Prec<F32>::io_t* __restrict__ k,
    const typename Prec<F32>::io_t* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, float scale, float* __restrict__ S,
    typename Prec<F32>::io_t* __restrict__ out, int64_t nbh) {
    using P = Prec<F32>;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t bh = (int64_t)blockIdx.x * 2 + (wv >> 1);
    if (bh >= nbh) return;  // whole wave: no barrier below
    const int half = wv & 1, cg = lane & 15, rg = lane >> 4;
    const int col = 64 * half + 4 * cg;

    float* Sb = S + bh * (kD * kD);
    f32x4 s[32];
#pragma unroll
    for (int m = 0; m < 32; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sb + (32 * rg + m) * kD + col));

    // per-wave copies of q, k and exp(g) (each wave reads what it wrote)
    __shared__ float lq[4][kD], lk[4][kD], la[4][kD];
    const float q0 = P::from_io(q[bh * kD + lane]), q1 = P::from_io(q[bh * kD + lane + 64]);
    const float k0 = P::from_io(k[bh * kD + lane]), k1 = P::from_io(k[bh * kD + lane + 64]);
    lq[wv][lane] = q0;
    lq[wv][lane + 64] = q1;
    lk[wv][lane] = k0;
    lk[wv][lane + 64] = k1;
    la[wv][lane] = fast_exp(g[bh * kD + lane]);
    la[wv][lane + 64] = fast_exp(g[bh * kD + lane + 64]);
    float ssq = q0 * q0 + q1 * q1, ssk = k0 * k0 + k1 * k1, sqk = q0 * k0 + q1 * k1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        ssq += __shfl_xor(ssq, off);
        ssk += __shfl_xor(ssk, off);
        sqk += __shfl_xor(sqk, off);
    }
    const float iq = 1.0f / sqrtf(ssq + kNormEps), ik = 1.0f / sqrtf(ssk + kNormEps);
    const float kq = sqk * iq * ik;
    const float bt = beta[bh];
    float vv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) vv[c] = P::from_io(v[bh * kD + col + c]);
    __builtin_amdgcn_wave_barrier();

    f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 32; ++m) {
        const int row = 32 * rg + m;
        const float a = la[wv][row], kk = lk[wv][row], qq = lq[wv][row];
        s[m] *= a;
        p += kk * s[m];
        r += qq * s[m];
    }
    // the four row groups of a column group sit at lanes cg, cg+16, cg+32, cg+48
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        p[c] += __shfl_xor(p[c], 16);
        p[c] += __shfl_xor(p[c], 32);
        r[c] += __shfl_xor(r[c], 16);
        r[c] += __shfl_xor(r[c], 32);
    }
    f32x4 u;
#pragma unroll
    for (int c = 0; c < 4; ++c) u[c] = bt * (vv[c] - p[c] * ik);
    if (rg == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) out[bh * kD + col + c] = P::to_io(scale * (r[c] * iq + kq * u[c]));
    }
#pragma unroll
    for (int m = 0; m < 32; ++m) {
        const float kk = lk[wv][32 * rg + m] * ik;
        s[m] += kk * u;
        __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4*>(Sb + (32 * rg + m) * kD + col));
    }
}

template <bool F32>
hipError_t launch_decode(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float scale, float* S, void* out, int B, int H,
                         hipStream_t stream) {
    using io = typename Prec<F32>::io_t;
    const int64_t nbh = (int64_t)B * H;
    const unsigned nblk = (unsigned)((nbh + 1) / 2);
    hipLaunchKernelGGL(kda_decode_kernel<F32>, dim3(nblk), dim3(256), 0, stream,
                       static_cast<const io*>(q), static_cast<const io*>(k),
                       static_cast<const io*>(v), g, beta, scale, S, static_cast<io*>(out), nbh);
    return hipGetLastError();
}

template hipError_t launch_decode<false>(const void*, const void*, const void*, const float*,
                                         const float*, float, float*, void*, int, int,
                                         hipStream_t);
template hipError_t launch_decode<true>(const void*, const void*, const void*, const float*,
                                        const float*, float, float*, void*, int, int,
                                        hipStream_t);

}  // namespace kda
