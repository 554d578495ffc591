// Backward of one recurrent KDA step (training through the recurrence, one
// token at a time in reverse), and its C entry points (fp32 and bf16 I/O).
//
// The step (Kimi-K3 深度解析 blog, section 三; 深入 Kimi-K3 thread, KDA
// paragraph, for the in-kernel L2 norms):
//   qh = q / |q|,  kh = k / |k|,  St = Diag(exp g) S_prev,  p = St^T kh,
//   u = beta (v - p),  S_new = St + kh u^T,  o = scale S_new^T qh.
// Given G = dL/dS_new and d_o = dL/do, reverse-mode differentiation of these
// assignments, in reverse order, gives (Gh = G + scale qh d_o^T):
//   dqh = scale (St d_o + kh (u . d_o))
//   du = Gh^T kh = G^T kh + scale (qh . kh) d_o,   dv = beta du,
//   dbeta = du . (v - p),   dp = -beta du
//   dkh = Gh u + St dp = G u + scale qh (d_o . u) + St dp
//   dSt = Gh + kh dp^T,   dS_prev = Diag(exp g) dSt,
//   dg_i = sum_j St_ij dSt_ij = (St . G)_i + scale qh_i (St d_o)_i + kh_i (St dp)_i
//   dq = (dqh - qh (qh . dqh)) / |q|, likewise dk,
// with |x| = sqrt(x . x + eps).  One pass over S_prev and G per (b, h): the
// step reads 128 KB and writes 64 KB of state gradient, an HBM stream like
// the forward decode step.
//
// Layout: one 256-thread workgroup per (b, h).  Wave w owns value columns
// 32w .. 32w+31 for all 128 key rows; lane (cg, rg) = (lane % 8, lane / 8)
// holds columns 32w + 4cg .. +3 of rows 16rg .. 16rg+15 of St and G, so the
// sums over key rows (p, G^T kh) stay inside the wave (lane sums and three
// xor shuffles); the sums over value columns are finished across the four
// waves in LDS.
#include <math.h>
#include <stdint.h>

#include "../../include/kda.h"
#include "kda_common.hpp"
#include "kda_debug.hpp"

namespace kda {
namespace {

// F32: q, k, v, dout, dq, dk, dv in fp32; else in bf16 (rounded to nearest
// even on store).  g, beta, the states and dg, dbeta are fp32 either way.
template <bool F32>
__global__ __launch_bounds__(256) void kda_step_bwd_kernel(
    const typename Prec<F32>::io_t* __restrict__ q, const typename Prec<F32>::io_t* __restrict__ k,
    const typename Prec<F32>::io_t* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, float scale, const float* __restrict__ S_prev,
    const typename Prec<F32>::io_t* __restrict__ d_o, float* __restrict__ dS,
    typename Prec<F32>::io_t* __restrict__ dq, typename Prec<F32>::io_t* __restrict__ dk,
    typename Prec<F32>::io_t* __restrict__ dv, float* __restrict__ dg,
    float* __restrict__ dbeta) {
    using P = Prec<F32>;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t bh = blockIdx.x;
    const int cg = lane & 7, rg = lane >> 3;
    const int col = 32 * w + 4 * cg, row0 = 16 * rg;
    __shared__ float qh_s[kD], kh_s[kD], a_s[kD];  // normalised q, k; exp(g)
    __shared__ float part_s[4][4][kD];             // per-wave row sums over its columns
    __shared__ float sc_s[2][4];                   // per-wave (u . d_o), (du . (v - p))
    __shared__ float dot_s[2][2];                  // (q . dqh), (k . dkh) per half of the rows

    // the state and its gradient: 16 rows x 4 columns of each per lane
    const float* Sb = S_prev + bh * (kD * kD);
    float* Gb = dS + bh * (kD * kD);
    f32x4 St[16], G[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        St[m] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(Sb + (row0 + m) * kD + col));
        G[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Gb + (row0 + m) * kD + col));
    }

    // norms (every wave computes them; wave 0 publishes qh, kh, exp g)
    const auto* qb = q + bh * kD;
    const auto* kb = k + bh * kD;
    const float q0 = P::from_io(qb[lane]), q1 = P::from_io(qb[lane + 64]);
    const float k0 = P::from_io(kb[lane]), k1 = P::from_io(kb[lane + 64]);
    float ssq = q0 * q0 + q1 * q1, ssk = k0 * k0 + k1 * k1, sqk = q0 * k0 + q1 * k1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        ssq += __shfl_xor(ssq, off);
        ssk += __shfl_xor(ssk, off);
        sqk += __shfl_xor(sqk, off);
    }
    const float rq = 1.0f / sqrtf(ssq + kNormEps), rk = 1.0f / sqrtf(ssk + kNormEps);
    const float qk = sqk * rq * rk;
    if (w == 0) {
        qh_s[lane] = q0 * rq;
        qh_s[lane + 64] = q1 * rq;
        kh_s[lane] = k0 * rk;
        kh_s[lane + 64] = k1 * rk;
        a_s[lane] = fast_exp(g[bh * kD + lane]);
        a_s[lane + 64] = fast_exp(g[bh * kD + lane + 64]);
    }
    const float bt = beta[bh];
    float vv[4], dov[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        vv[c] = P::from_io(v[bh * kD + col + c]);
        dov[c] = P::from_io(d_o[bh * kD + col + c]);
    }
    __syncthreads();

    // decay the rows; sums over the key rows: p = St^T kh, ag = G^T kh
    f32x4 p = {0.f, 0.f, 0.f, 0.f}, ag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int i = row0 + m;
        const float kk = kh_s[i];
        St[m] *= a_s[i];
        p += kk * St[m];
        ag += kk * G[m];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int off = 8; off <= 32; off <<= 1) {
            p[c] += __shfl_xor(p[c], off);
            ag[c] += __shfl_xor(ag[c], off);
        }
    }
    // per value column
    float u[4], du[4], dp[4], ud = 0.f, db = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        u[c] = bt * (vv[c] - p[c]);
        du[c] = ag[c] + scale * qk * dov[c];
        dp[c] = -bt * du[c];
        ud += u[c] * dov[c];
        db += du[c] * (vv[c] - p[c]);
    }
    if (rg == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) dv[bh * kD + col + c] = P::to_io(bt * du[c]);
    }
#pragma unroll
    for (int off = 1; off <= 4; off <<= 1) {
        ud += __shfl_xor(ud, off);
        db += __shfl_xor(db, off);
    }
    if (lane == 0) {
        sc_s[0][w] = ud;
        sc_s[1][w] = db;
    }

    // sums over this wave's 32 value columns for each key row: St d_o,
    // G u, St dp, St . G
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        float x = 0.f, gu = 0.f, z = 0.f, sg = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            x += St[m][c] * dov[c];
            gu += G[m][c] * u[c];
            z += St[m][c] * dp[c];
            sg += St[m][c] * G[m][c];
        }
#pragma unroll
        for (int off = 1; off <= 4; off <<= 1) {
            x += __shfl_xor(x, off);
            gu += __shfl_xor(gu, off);
            z += __shfl_xor(z, off);
            sg += __shfl_xor(sg, off);
        }
        if (cg == 0) {
            part_s[0][w][row0 + m] = x;
            part_s[1][w][row0 + m] = gu;
            part_s[2][w][row0 + m] = z;
            part_s[3][w][row0 + m] = sg;
        }
    }

    // dS_prev = exp(g_i) (G + scale qh_i d_o^T + kh_i dp^T), over G in place
    // (each lane rewrites only what it read)
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int i = row0 + m;
        const float qq = scale * qh_s[i], kk = kh_s[i], a = a_s[i];
        f32x4 y;
#pragma unroll
        for (int c = 0; c < 4; ++c) y[c] = a * (G[m][c] + qq * dov[c] + kk * dp[c]);
        __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(Gb + (row0 + m) * kD + col));
    }
    __syncthreads();

    // per key row (threads 0..127): dqh, dkh, dg; then the norms' backward
    float dqh = 0.f, dkh = 0.f;
    const int i = tid & (kD - 1);
    if (tid < kD) {
        const float x = part_s[0][0][i] + part_s[0][1][i] + part_s[0][2][i] + part_s[0][3][i];
        const float gu = part_s[1][0][i] + part_s[1][1][i] + part_s[1][2][i] + part_s[1][3][i];
        const float z = part_s[2][0][i] + part_s[2][1][i] + part_s[2][2][i] + part_s[2][3][i];
        const float sg = part_s[3][0][i] + part_s[3][1][i] + part_s[3][2][i] + part_s[3][3][i];
        const float uds = sc_s[0][0] + sc_s[0][1] + sc_s[0][2] + sc_s[0][3];
        const float qq = qh_s[i], kk = kh_s[i];
        dqh = scale * (x + kk * uds);
        dkh = gu + scale * qq * uds + z;
        dg[bh * kD + i] = sg + scale * qq * x + kk * z;
        if (tid == 0) dbeta[bh] = sc_s[1][0] + sc_s[1][1] + sc_s[1][2] + sc_s[1][3];
    }
    // (qh . dqh) and (kh . dkh) over the 128 rows: waves 0 and 1
    float tq = tid < kD ? qh_s[i] * dqh : 0.f, tk = tid < kD ? kh_s[i] * dkh : 0.f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        tq += __shfl_xor(tq, off);
        tk += __shfl_xor(tk, off);
    }
    if (lane == 0 && w < 2) {
        dot_s[0][w] = tq;
        dot_s[1][w] = tk;
    }
    __syncthreads();
    if (tid < kD) {
        const float qdq = dot_s[0][0] + dot_s[0][1], kdk = dot_s[1][0] + dot_s[1][1];
        dq[bh * kD + i] = P::to_io(rq * (dqh - qh_s[i] * qdq));
        dk[bh * kD + i] = P::to_io(rk * (dkh - kh_s[i] * kdk));
    }
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace
}  // namespace kda

namespace {

template <bool F32>
kda_status_t step_bwd(const void* q, const void* k, const void* v, const float* g,
                      const float* beta, float scale, const float* S_prev, const void* dout,
                      float* dS, void* dq, void* dk, void* dv, float* dg, float* dbeta, int B,
                      int H, hipStream_t stream) {
    using kda::aligned;
    using kda::overlap;
    using io = typename kda::Prec<F32>::io_t;
    if (B < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    if (B == 0 || H == 0) return KDA_OK;
    const void* ins[] = {q, k, v, g, S_prev, dout};
    const void* outs[] = {dq, dk, dv, dg};
    for (const void* p : ins)
        if (!p || !aligned(p, 16)) return KDA_ERR_INVALID_ARG;
    for (const void* p : outs)
        if (!p || !aligned(p, 16)) return KDA_ERR_INVALID_ARG;
    if (!dS || !aligned(dS, 16) || !beta || !aligned(beta, 4) || !dbeta || !aligned(dbeta, 4))
        return KDA_ERR_INVALID_ARG;
    if ((int64_t)B * H > ((int64_t)1 << 31) - 1) return KDA_ERR_UNSUPPORTED;
    const size_t nbh = (size_t)B * H;
    const size_t vec = nbh * KDA_HEAD_DIM * sizeof(io);      // q, k, v, dout, dq, dk, dv
    const size_t vec32 = nbh * KDA_HEAD_DIM * sizeof(float);  // g, dg
    const size_t sbytes = vec32 * KDA_HEAD_DIM;
    const size_t ins_n[] = {vec, vec, vec, vec32, sbytes, vec};
    // every written buffer overlaps nothing else that is read or written
    const void* written[] = {dq, dk, dv, dg, dbeta, dS};
    const size_t written_n[] = {vec, vec, vec, vec32, nbh * sizeof(float), sbytes};
    for (int a = 0; a < 6; ++a) {
        for (int b = 0; b < 6; ++b)
            if (overlap(written[a], written_n[a], ins[b], ins_n[b])) return KDA_ERR_INVALID_ARG;
        if (overlap(written[a], written_n[a], beta, nbh * sizeof(float)))
            return KDA_ERR_INVALID_ARG;
        for (int b = a + 1; b < 6; ++b)
            if (overlap(written[a], written_n[a], written[b], written_n[b]))
                return KDA_ERR_INVALID_ARG;
    }
    kda::DebugScope dbg(stream);
    if (dbg.on()) {
        if (dbg.setup_status() != KDA_OK) return dbg.setup_status();
        const size_t nel = nbh * KDA_HEAD_DIM;
        dbg.finite(static_cast<const io*>(q), nel);
        dbg.finite(static_cast<const io*>(k), nel);
        dbg.finite(static_cast<const io*>(v), nel);
        dbg.finite(static_cast<const io*>(dout), nel);
        dbg.decay(g, nel);
        dbg.finite(beta, nbh);
        dbg.finite(S_prev, nel * KDA_HEAD_DIM);
        dbg.finite(dS, nel * KDA_HEAD_DIM);
        const kda_status_t st = dbg.inputs_status();
        if (st != KDA_OK) return st;
    }
    hipLaunchKernelGGL(kda::kda_step_bwd_kernel<F32>, dim3((unsigned)nbh), dim3(256), 0, stream,
                       static_cast<const io*>(q), static_cast<const io*>(k),
                       static_cast<const io*>(v), g, beta, scale, S_prev,
                       static_cast<const io*>(dout), dS, static_cast<io*>(dq),
                       static_cast<io*>(dk), static_cast<io*>(dv), dg, dbeta);
    if (hipGetLastError() != hipSuccess) return KDA_ERR_HIP;
    return dbg.on() ? dbg.device_status() : KDA_OK;
}

}  // namespace

extern "C" kda_status_t kda_recurrent_step_bwd_f32(
    const float* q, const float* k, const float* v, const float* g, const float* beta,
    float scale, const float* S_prev, const float* dout, float* dS, float* dq, float* dk,
    float* dv, float* dg, float* dbeta, int B, int H, hipStream_t stream) {
    return step_bwd<true>(q, k, v, g, beta, scale, S_prev, dout, dS, dq, dk, dv, dg, dbeta, B, H,
                          stream);
}

extern "C" kda_status_t kda_recurrent_step_bwd(
    const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g, const float* beta,
    float scale, const float* S_prev, const uint16_t* dout, float* dS, uint16_t* dq,
    uint16_t* dk, uint16_t* dv, float* dg, float* dbeta, int B, int H, hipStream_t stream) {
    return step_bwd<false>(q, k, v, g, beta, scale, S_prev, dout, dS, dq, dk, dv, dg, dbeta, B,
                           H, stream);
}
