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
//
// CONV: q, k and v arrive raw and first pass through the 4-tap causal short
// convolution + SiLU that the KDA layer puts in front of the attention (深入
// Kimi-K3 thread, KDA paragraph; kernel size 4 in the Kimi K3 architecture
// page's config table), with the 3 previous raw tokens of each (b, h) taken
// from the conv state, which the step then advances by one token in place.
// Both waves of a (b, h) read the q / k rows of that state, so it is written
// only after a workgroup barrier; every wave reaches it (a wave past the end
// computes on a valid (b, h) and stores nothing).  An optional output gate
// multiplies o by sigmoid of its logits before the store.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

// silu(sum_j w[j] x_{t-3+j}) for one channel: x3 is the current raw token,
// st the three before it (oldest first), rounded to bf16 as the attention
// input; the same arithmetic, in the same order, as the prefill's filter
__device__ __forceinline__ float conv_silu1(f32x4 w, const float* st, float x3) {
    float acc = 0.f;
    acc += w[0] * st[0];
    acc += w[1] * st[1];
    acc += w[2] * st[2];
    acc += w[3] * x3;
    const float y = acc * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * acc));
    return bf2f(f2bf(y));
}

}  // namespace

template <bool F32, bool CONV>
__global__ __launch_bounds__(256) void kda_decode_kernel(
    const typename Prec<F32>::io_t* __restrict__ q, const typename Prec<F32>::io_t* __restrict__ k,
    const typename Prec<F32>::io_t* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, float scale, float* __restrict__ S,
    typename Prec<F32>::io_t* __restrict__ out, int64_t nbh, DecodeConv conv) {
    using P = Prec<F32>;
    static_assert(!(CONV && F32), "the short convolution is offered with bf16 I/O only");
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int64_t bh = (int64_t)blockIdx.x * 2 + (wv >> 1);
    const bool live = bh < nbh;
    if constexpr (!CONV) {
        if (!live) return;  // whole wave: no barrier below
    } else {
        if (!live) bh = nbh - 1;  // compute on a valid (b, h), store nothing
    }
    const int half = wv & 1, cg = lane & 15, rg = lane >> 4;
    const int col = 64 * half + 4 * cg;

    float* Sb = S + bh * (kD * kD);
    f32x4 s[32];
#pragma unroll
    for (int m = 0; m < 32; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sb + (32 * rg + m) * kD + col));

    // per-wave copies of q, k and exp(g) (each wave reads what it wrote)
    __shared__ float lq[4][kD], lk[4][kD], la[4][kD];
    float q0, q1, k0, k1;
    // conv state rows of this (b, h): tensor x (q 0, k 1, v 2), token j
    // (0 = oldest) at cs(x, j) + channel
    uint16_t* cs0 = nullptr;
    int64_t cs_ten = 0, cs_tok = 0;
    float sq[2][3], sk[2][3], sv[4][3];
    if constexpr (CONV) {
        const int64_t H = conv.H, b = bh / H, h = bh % H;
        cs_tok = H * kD;
        cs_ten = (int64_t)conv.B * 3 * cs_tok;
        cs0 = conv.state + (b * 3 * H + h) * kD;
        const int ch[2] = {lane, lane + 64};
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                sq[e][j] = bf2f(cs0[j * cs_tok + ch[e]]);
                sk[e][j] = bf2f(cs0[cs_ten + j * cs_tok + ch[e]]);
            }
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int j = 0; j < 3; ++j) sv[c][j] = bf2f(cs0[2 * cs_ten + j * cs_tok + col + c]);
        float xq[2], xk[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            xq[e] = bf2f(q[bh * kD + ch[e]]);
            xk[e] = bf2f(k[bh * kD + ch[e]]);
            const f32x4 wqe = *reinterpret_cast<const f32x4*>(conv.wq + (h * kD + ch[e]) * 4);
            const f32x4 wke = *reinterpret_cast<const f32x4*>(conv.wk + (h * kD + ch[e]) * 4);
            const float yq = conv_silu1(wqe, sq[e], xq[e]);
            const float yk = conv_silu1(wke, sk[e], xk[e]);
            // the state rows move one token on: drop the oldest, append raw x
            sq[e][0] = sq[e][1];
            sq[e][1] = sq[e][2];
            sq[e][2] = xq[e];
            sk[e][0] = sk[e][1];
            sk[e][1] = sk[e][2];
            sk[e][2] = xk[e];
            if (e == 0) {
                q0 = yq;
                k0 = yk;
            } else {
                q1 = yq;
                k1 = yk;
            }
        }
    } else {
        q0 = P::from_io(q[bh * kD + lane]);
        q1 = P::from_io(q[bh * kD + lane + 64]);
        k0 = P::from_io(k[bh * kD + lane]);
        k1 = P::from_io(k[bh * kD + lane + 64]);
    }
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
    if constexpr (CONV) {
        const int64_t h = bh % conv.H;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float xv = bf2f(v[bh * kD + col + c]);
            const f32x4 wve = *reinterpret_cast<const f32x4*>(conv.wv + (h * kD + col + c) * 4);
            vv[c] = conv_silu1(wve, sv[c], xv);
            sv[c][0] = sv[c][1];
            sv[c][1] = sv[c][2];
            sv[c][2] = xv;
        }
        // both waves of this (b, h) have read its conv state: advance it
        __syncthreads();
        if (live) {
            if (half == 0) {
                const int ch[2] = {lane, lane + 64};
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int j = 0; j < 3; ++j) {
                        cs0[j * cs_tok + ch[e]] = f2bf(sq[e][j]);
                        cs0[cs_ten + j * cs_tok + ch[e]] = f2bf(sk[e][j]);
                    }
            }
            if (rg == 0) {
#pragma unroll
                for (int j = 0; j < 3; ++j)
                    *reinterpret_cast<uint2*>(cs0 + 2 * cs_ten + j * cs_tok + col) =
                        uint2{(uint32_t)f2bf(sv[0][j]) | ((uint32_t)f2bf(sv[1][j]) << 16),
                              (uint32_t)f2bf(sv[2][j]) | ((uint32_t)f2bf(sv[3][j]) << 16)};
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) vv[c] = P::from_io(v[bh * kD + col + c]);
    }
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
    if (CONV && !live) return;
    if (rg == 0) {
        float gt[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (CONV) {
            if (conv.gate) {
                // the output gate: out = o * sigmoid(z)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    gt[c] = __builtin_amdgcn_rcpf(
                        1.f + __builtin_amdgcn_exp2f(-kLog2e * bf2f(conv.gate[bh * kD + col + c])));
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float y = scale * (r[c] * iq + kq * u[c]);
            if constexpr (CONV) y *= gt[c];
            out[bh * kD + col + c] = P::to_io(y);
        }
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
                         const DecodeConv* conv, hipStream_t stream) {
    using io = typename Prec<F32>::io_t;
    const int64_t nbh = (int64_t)B * H;
    const unsigned nblk = (unsigned)((nbh + 1) / 2);
    if constexpr (!F32) {
        if (conv) {
            hipLaunchKernelGGL((kda_decode_kernel<false, true>), dim3(nblk), dim3(256), 0, stream,
                               static_cast<const io*>(q), static_cast<const io*>(k),
                               static_cast<const io*>(v), g, beta, scale, S,
                               static_cast<io*>(out), nbh, *conv);
            return hipGetLastError();
        }
    } else {
        if (conv) return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL((kda_decode_kernel<F32, false>), dim3(nblk), dim3(256), 0, stream,
                       static_cast<const io*>(q), static_cast<const io*>(k),
                       static_cast<const io*>(v), g, beta, scale, S, static_cast<io*>(out), nbh,
                       DecodeConv{});
    return hipGetLastError();
}

template hipError_t launch_decode<false>(const void*, const void*, const void*, const float*,
                                         const float*, float, float*, void*, int, int,
                                         const DecodeConv*, hipStream_t);
template hipError_t launch_decode<true>(const void*, const void*, const void*, const float*,
                                        const float*, float, float*, void*, int, int,
                                        const DecodeConv*, hipStream_t);

}  // namespace kda
