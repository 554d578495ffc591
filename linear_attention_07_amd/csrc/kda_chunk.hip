// Chunkwise-parallel KDA prefill (the pages' chunk_kda) for fp32 q/k/v/o, in
// fp32 arithmetic (prep: 16x16x4 fp32 matrix-core products; scan: bf16
// products of hi / lo pairs, fp32-like).  bf16 inputs take the kernels of
// kda_chunk16.hip.
//
// The recurrence (Kimi-K3 深度解析 blog, section 三) is evaluated 64 tokens at a
// time.  The chunk form below is an exact rearrangement of it; the blog's
// "Triton 实现" paragraph describes a chunked kernel with an inner-chunk part and
// a cross-chunk part, and the ai-pulse-lab summary of the technical report
// (architecture section) explains why the -5 lower bound on the log-decay is
// what lets the diagonal blocks run as dense matrix-core products.
//
// For one (batch, head) and one chunk of tokens r = 0..63 entering with state S
// (key channel x value channel), let Gam_r = sum_{s<=r} g_s (per channel), and
//   Kt_r = exp(Gam_r) * kh_r       Qt_r = exp(Gam_r) * qh_r
//   Kb_r = exp(Gam_63 - Gam_r) * kh_r,   gamma = exp(Gam_63)
//   (KK)_ri = sum_c kh_rc kh_ic exp(Gam_rc - Gam_ic),  (QK)_ri likewise with qh_r
//   A = strict-lower(diag(beta) KK),  M = lower-incl(QK)
//   T = (I + A)^-1 diag(beta)                              (UT / WY form)
//   W = T Kt,   Q' = Qt - M W,   MT = M T.
// Token by token the errors u_r = beta_r (v_r - prediction_r) stack into
//   U = T V - W S,
//   O = scale (Qt S + M U) = scale (Q' S + MT V),
//   S <- Diag(gamma) S + Kb^T U.
//
// Range of the decay factors.  exp(Gam_r - Gam_i) is formed as a product of a
// row factor and a column factor about a reference token.  The reference for
// the 16-token column block b is its last token e_b = 16b + 15:
//   column factor exp(Gam_{e_b} - Gam_i) <= 1 for every i in block b,
//   row factor    exp(Gam_r - Gam_{e_b}) <= 1 for r in a later block,
//                 in [1, exp(75)] for r in block b itself (15 steps of at most
//                 5 each): finite in fp32 and bf16 because g >= -5.
// Values that underflow are bounded by the true (tiny) products.
//
// Precision.  The prep's operands and products are fp32 (the in-chunk inverse
// included).  The scan splits every operand into a bf16 hi + lo pair (x = hi +
// lo to about 2^-18 relative) and takes three bf16 products per pair, about
// 1e-5 relative per product, accumulated in fp32, with the state in fp32.
//
// Two kernels:
//   prep (one workgroup per chunk, fully parallel) computes W, Q', Kb^T, T, MT
//        and gamma from q, k, g, beta and writes them to a per-chunk record;
//   scan (one workgroup per head and 64 value columns) walks the chunks in
//        order with its slice of S in registers, on matrix cores, its loader
//        waves staging each record in LDS as operand fragments.
#include "kda_bf16.hpp"
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace {

using P = Prec<true>;
using F8 = P::F8;
using F4 = P::F4;

using RecF = ChunkRecF32;

constexpr int kScanSlices = 2;          // value-column slices per head
constexpr int kSliceCols = kD / kScanSlices;

}  // namespace

size_t chunk_f32_record_bytes() { return RecF::BYTES; }
int chunk_f32_slices() { return kScanSlices; }

// ---------------------------------------------------------------------------
// prep: one workgroup = one chunk of one (b, h).  Wave a owns chunk rows
// 16a..16a+15; lane (n = lane%16, g = lane/16) owns row 16a+n and the 32
// channels 32s + 8g + e (s, e = 0..3, 0..7), i.e. exactly the A-operand
// fragment of that row for the four k32 steps over the 128 channels.
// ---------------------------------------------------------------------------
// IO: float, or uint16_t for bf16 q and k (the backward of the bf16 prefill)
template <typename IO>
__global__ __launch_bounds__(256, 2) void kda_chunk_prep_kernel(
    const IO* __restrict__ q, const IO* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, int T, int H, int chunk0, int nchunks,
    uint8_t* __restrict__ ws, float* __restrict__ x_out) {
    using st = float;
    using R = RecF;

    const int cl = blockIdx.x % nchunks;
    const int bh = blockIdx.x / nchunks;
    const int h = bh % H, b = bh / H;
    const int c = chunk0 + cl;
    const int L = min(kChunk, T - c * kChunk);
    uint8_t* rec = ws + ((size_t)bh * nchunks + cl) * R::BYTES;
    st* Wg = reinterpret_cast<st*>(rec + R::W);
    st* QPg = reinterpret_cast<st*>(rec + R::QP);
    st* KTg = reinterpret_cast<st*>(rec + R::KT);
    st* THg = reinterpret_cast<st*>(rec + R::TH);
    st* MHg = reinterpret_cast<st*>(rec + R::MH);
    float* Gg = reinterpret_cast<float*>(rec + R::G);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;
    const int r = 16 * wv + n;
    const bool valid = r < L;
    const int64_t tok = (int64_t)c * kChunk + r;
    const int64_t rowoff = (((int64_t)b * T + tok) * H + h) * kD;

    constexpr int SP = kChunk + 1;   // fp32 pitch of the 64 x 64 matrices
    constexpr int KTP = kD + 4;      // pitch of the Kt rows (st elements)
    constexpr int MWP = kD + 4;      // fp32 pitch of the M W rows
    constexpr size_t kZfBytes = sizeof(F8) * 4 * 4 * 64;
    constexpr size_t kXBytes = sizeof(float) * kChunk * SP;
    constexpr size_t kKtBytes = (sizeof(st) * kChunk * KTP + 15) / 16 * 16;
    constexpr size_t kABytes = sizeof(float) * kChunk * SP;
    constexpr size_t kMwBytes = sizeof(float) * kChunk * MWP;
    // One area, so that two workgroups fit on a CU (77 KB of LDS each): the
    // KK / QK column operands, then X over them, with A after them; Kt after X
    // once A is dead (after the inverse); M W over Kt once W is formed.
    constexpr size_t kAOff = kZfBytes;
    constexpr size_t kKtOff = (kXBytes + 15) / 16 * 16;
    constexpr size_t kKtMw = kKtBytes > kMwBytes ? kKtBytes : kMwBytes;
    constexpr size_t kAreaBytes =
        kAOff + kABytes > kKtOff + kKtMw ? kAOff + kABytes : kKtOff + kKtMw;
    static_assert(kXBytes <= kAOff, "X lies within the column operands' space");
    // decay tables per channel (exp of sums of block totals tau_a):
    //   EP_a = exp(sum_{a'<a} tau), EK_a = exp(sum_{a'>a} tau), IE_a = exp(-tau_a),
    //   TF(a,b) = exp(sum_{b<a'<a} tau) for a - b >= 2: (2,0), (3,0), (3,1)
    enum { kEP = 0, kEK = 4, kIE = 8, kTF20 = 12, kTF30 = 13, kTF31 = 14, kTabs = 15 };
    __shared__ float tau_s[4][kD];
    __shared__ __align__(16) float tab_s[kTabs][kD];
    __shared__ float beta_s[kChunk];
    __shared__ float m_s[kChunk * SP];
    __shared__ __align__(16) uint8_t area[kAreaBytes];
    F8(*zf_s)[4][64] = reinterpret_cast<F8(*)[4][64]>(area);  // KK / QK column operands
    float* x_s = reinterpret_cast<float*>(area);              // X, then T = X diag(beta)
    float* a_s = reinterpret_cast<float*>(area + kAOff);      // diag(beta) strict-lower KK
    st* kt_s = reinterpret_cast<st*>(area + kKtOff);          // Kt
    float* mw_s = reinterpret_cast<float*>(area + kKtOff);    // M W

    // ---- load the lane's row: 32 channels of q, k, g -----------------------
    float qf[32], kf[32], lam[32];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int cb = 32 * s + 8 * gq;
        if (valid) {
            load8(q + rowoff + cb, qf + 8 * s);
            load8(k + rowoff + cb, kf + 8 * s);
            load8(g + rowoff + cb, lam + 8 * s);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[8 * s + e] = kf[8 * s + e] = lam[8 * s + e] = 0.f;
        }
    }
    const float bet = valid ? beta[((int64_t)b * T + tok) * H + h] : 0.f;

    // ---- L2 normalisation of q and k (row spread over lanes n, n+16, +32, +48)
    float ssq = 0.f, ssk = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        ssq += qf[j] * qf[j];
        ssk += kf[j] * kf[j];
    }
    ssq += __shfl_xor(ssq, 16);
    ssk += __shfl_xor(ssk, 16);
    ssq += __shfl_xor(ssq, 32);
    ssk += __shfl_xor(ssk, 32);
    const float iq = 1.0f / sqrtf(ssq + kNormEps), ik = 1.0f / sqrtf(ssk + kNormEps);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        qf[j] *= iq;
        kf[j] *= ik;
    }

    // ---- in-block inclusive cumsum of g over the 16 rows (lanes of a DPP row)
#pragma unroll
    for (int j = 0; j < 32; ++j) lam[j] = row16_inclusive_scan(lam[j]);
    if (n == 15) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) tau_s[wv][32 * s + 8 * gq + e] = lam[8 * s + e];
    }
    if (gq == 0) beta_s[r] = bet;
    __syncthreads();

    for (int idx = tid; idx < (kTabs + 1) * kD; idx += 256) {
        const int tb = idx >> 7, ch = idx & 127;
        const float t0 = tau_s[0][ch], t1 = tau_s[1][ch], t2 = tau_s[2][ch], t3 = tau_s[3][ch];
        float x;
        switch (tb) {
            case kEP + 0: x = 0.f; break;
            case kEP + 1: x = t0; break;
            case kEP + 2: x = t0 + t1; break;
            case kEP + 3: x = t0 + t1 + t2; break;
            case kEK + 0: x = t1 + t2 + t3; break;
            case kEK + 1: x = t2 + t3; break;
            case kEK + 2: x = t3; break;
            case kEK + 3: x = 0.f; break;
            case kIE + 0: x = -t0; break;
            case kIE + 1: x = -t1; break;
            case kIE + 2: x = -t2; break;
            case kIE + 3: x = -t3; break;
            case kTF20: x = t1; break;
            case kTF30: x = t1 + t2; break;
            case kTF31: x = t2; break;
            default: x = t0 + t1 + t2 + t3; break;  // chunk decay gamma
        }
        const float ex = fast_exp(x);
        if (tb < kTabs) tab_s[tb][ch] = ex;
        else Gg[ch] = ex;
    }
    __syncthreads();

    // ---- decay factors and the derived operands -----------------------------
    // e0 = exp(Gam_r - Gam_{16a-1}) <= 1, z = exp(Gam_{e_a} - Gam_r) <= 1
    // (a = this wave's block).  Kept: rk0 = kh e0, rq0 = qh e0, Qt.
    float qtil[32];
    {
        float zc[32];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int cb = 32 * s + 8 * gq;
            float ep[8], ek[8], ta[8];
            *reinterpret_cast<float4*>(ep) = *reinterpret_cast<const float4*>(&tab_s[kEP + wv][cb]);
            *reinterpret_cast<float4*>(ep + 4) = *reinterpret_cast<const float4*>(&tab_s[kEP + wv][cb + 4]);
            *reinterpret_cast<float4*>(ek) = *reinterpret_cast<const float4*>(&tab_s[kEK + wv][cb]);
            *reinterpret_cast<float4*>(ek + 4) = *reinterpret_cast<const float4*>(&tab_s[kEK + wv][cb + 4]);
#pragma unroll
            for (int e = 0; e < 8; ++e) ta[e] = tau_s[wv][cb + e];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = 8 * s + e;
                const float e0 = fast_exp(lam[j]);
                const float z = fast_exp(ta[e] - lam[j]);
                zc[j] = kf[j] * z;
                KTg[(size_t)(cb + e) * kChunk + r] = kf[j] * z * ek[e];
                qtil[j] = qf[j] * e0 * ep[e];
                kf[j] *= e0;  // rk0
                qf[j] *= e0;  // rq0
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) zf_s[wv][s][lane] = P::pack8(zc + 8 * s);
    }
    __syncthreads();

    // ---- (KK) and (QK) tiles of row block wv against column blocks cb <= wv -
    // row factor exp(Gam_r - Gam_{e_cb}) = e0 * f_cb with f = IE_wv (cb = wv),
    // 1 (cb = wv - 1), TF(wv, cb) otherwise
    for (int cb = 0; cb <= wv; ++cb) {
        const int tix = (cb == wv) ? kIE + wv : (wv - cb == 2) ? (wv == 2 ? kTF20 : kTF31) : kTF30;
        const bool unit = (cb == wv - 1);
        f32x4 accK = {0.f, 0.f, 0.f, 0.f}, accQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int cbase = 32 * s + 8 * gq;
            float f[8];
            if (unit) {
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = 1.f;
            } else {
                *reinterpret_cast<float4*>(f) = *reinterpret_cast<const float4*>(&tab_s[tix][cbase]);
                *reinterpret_cast<float4*>(f + 4) = *reinterpret_cast<const float4*>(&tab_s[tix][cbase + 4]);
            }
            float rk[8], rq[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                rk[e] = kf[8 * s + e] * f[e];
                rq[e] = qf[8 * s + e] * f[e];
            }
            const F8 fz = zf_s[cb][s][lane];
            accK = P::mma32(accK, P::pack8(rk), fz);
            accQ = P::mma32(accQ, P::pack8(rq), fz);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ri = 16 * wv + 4 * gq + e, ci = 16 * cb + n;
            const bool strict = (cb < wv) || (ci < ri);
            const bool incl = (cb < wv) || (ci <= ri);
            a_s[ri * SP + ci] = strict ? (x_out ? accK[e] : beta_s[ri] * accK[e]) : 0.f;
            m_s[ri * SP + ci] = incl ? accQ[e] : 0.f;
        }
    }
    __syncthreads();
    if (x_out) {
        // P = strict-lower(KK) and N = M, whole [64][64] (zero above the
        // diagonal blocks), after X in the chunk's slot; then A = diag(beta) P
        float* pg = x_out + (((size_t)bh * nchunks + cl) * 3 + 1) * kChunk * kChunk;
        float* ng = pg + kChunk * kChunk;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tid + 256 * j, rr = e >> 4, c4 = 4 * (e & 15);
            const bool low = (c4 >> 4) <= (rr >> 4);
            float pa[4], na[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                pa[u] = low ? a_s[rr * SP + c4 + u] : 0.f;
                na[u] = low ? m_s[rr * SP + c4 + u] : 0.f;
            }
            *reinterpret_cast<float4*>(pg + rr * kChunk + c4) = make_float4(pa[0], pa[1], pa[2], pa[3]);
            *reinterpret_cast<float4*>(ng + rr * kChunk + c4) = make_float4(na[0], na[1], na[2], na[3]);
            const float bt = beta_s[rr];
#pragma unroll
            for (int u = 0; u < 4; ++u) a_s[rr * SP + c4 + u] = pa[u] * bt;
        }
        __syncthreads();
    }

    // ---- X = (I + A)^-1: diagonal blocks by forward substitution (fp32) ----
    {
        float arow[16];
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
#pragma unroll
            for (int cc = 0; cc < rr; ++cc) arow[cc] = a_s[(16 * wv + rr) * SP + 16 * wv + cc];
            float s = 0.f;
#pragma unroll
            for (int cc = 0; cc < rr; ++cc) s += arow[cc] * x[cc];
            x[rr] = (rr == n) ? 1.f : -s;
        }
        if (gq == 0) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) x_s[(16 * wv + rr) * SP + 16 * wv + n] = x[rr];
        }
    }
    __syncthreads();
    // off-diagonal blocks by distance: X_ab = -X_aa sum_{c=b}^{a-1} A_ac X_cb
    for (int d = 1; d < 4; ++d) {
        if (wv >= d) {
            const int a = wv, bb = wv - d;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int cc = bb; cc < a; ++cc) {
                F4 fa, fb;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    fa.v[e] = a_s[(16 * a + n) * SP + 16 * cc + 4 * gq + e];
                    fb.v[e] = x_s[(16 * cc + 4 * gq + e) * SP + 16 * bb + n];
                }
                acc = P::mma16(acc, fa, fb);
            }
            F4 fx;
#pragma unroll
            for (int e = 0; e < 4; ++e) fx.v[e] = x_s[(16 * a + n) * SP + 16 * a + 4 * gq + e];
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            const f32x4 xab = P::mma16(zero, fx, P::pack4(acc));
#pragma unroll
            for (int e = 0; e < 4; ++e) x_s[(16 * a + 4 * gq + e) * SP + 16 * bb + n] = -xab[e];
        }
        __syncthreads();
    }
    // T = X diag(beta), zero above the diagonal (and X itself, if asked for)
    float* xg = x_out ? x_out + ((size_t)bh * nchunks + cl) * 3 * kChunk * kChunk : nullptr;
    for (int idx = tid; idx < kChunk * kChunk; idx += 256) {
        const int rr = idx >> 6, cc = idx & 63;
        if (xg) xg[idx] = (cc <= rr) ? x_s[rr * SP + cc] : 0.f;
        const float tv = (cc <= rr) ? x_s[rr * SP + cc] * beta_s[cc] : 0.f;
        x_s[rr * SP + cc] = tv;
        THg[idx] = tv;
    }
    // Kt = rk0 EP over the space of A, which the inverse no longer reads
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int cb = 32 * s + 8 * gq;
        float ep[8];
        *reinterpret_cast<float4*>(ep) = *reinterpret_cast<const float4*>(&tab_s[kEP + wv][cb]);
        *reinterpret_cast<float4*>(ep + 4) = *reinterpret_cast<const float4*>(&tab_s[kEP + wv][cb + 4]);
        st* dst = kt_s + r * KTP + cb;
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = kf[8 * s + e] * ep[e];
    }
    __syncthreads();

    // ---- W = T Kt for channels [32 wv, 32 wv + 32) ---------------------------
    f32x4 Wt[4][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int col = 32 * wv + 16 * ct + n;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb <= rt; ++kb) {
                f32x4 ta;
                F4 kv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ta[e] = x_s[(16 * rt + n) * SP + 16 * kb + 4 * gq + e];
                    kv.v[e] = kt_s[(16 * kb + 4 * gq + e) * KTP + col];
                }
                acc = P::mma16(acc, P::pack4(ta), kv);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Wt[rt][ct][e] = acc[e];
                Wg[(size_t)(16 * rt + 4 * gq + e) * kD + col] = acc[e];
            }
        }
    }

    // ---- MT = M T, row block wv (for the forward scan only: the backward,
    // which asks for X, reads no MT) ------------------------------------------
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        if (x_out) break;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int kb = ct; kb <= wv; ++kb) {
            f32x4 ma, tb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ma[e] = m_s[(16 * wv + n) * SP + 16 * kb + 4 * gq + e];
                tb[e] = x_s[(16 * kb + 4 * gq + e) * SP + 16 * ct + n];
            }
            acc = P::mma16(acc, P::pack4(ma), P::pack4(tb));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) MHg[(size_t)(16 * wv + 4 * gq + e) * kChunk + 16 * ct + n] = acc[e];
    }
    __syncthreads();  // Kt and A are dead: their space takes M W

    // ---- M W for channels [32 wv, 32 wv + 32), then Q' = Qt - M W per row ---
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int col = 32 * wv + 16 * ct + n;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb <= rt; ++kb) {
                f32x4 ma;
#pragma unroll
                for (int e = 0; e < 4; ++e) ma[e] = m_s[(16 * rt + n) * SP + 16 * kb + 4 * gq + e];
                acc = P::mma16(acc, P::pack4(ma), P::pack4(Wt[kb][ct]));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) mw_s[(16 * rt + 4 * gq + e) * MWP + col] = acc[e];
        }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int cb = 32 * s + 8 * gq;
        float mw[8];
        *reinterpret_cast<float4*>(mw) = *reinterpret_cast<const float4*>(&mw_s[r * MWP + cb]);
        *reinterpret_cast<float4*>(mw + 4) = *reinterpret_cast<const float4*>(&mw_s[r * MWP + cb + 4]);
        float o8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] = qtil[8 * s + e] - mw[e];
        float* dst = QPg + (size_t)r * kD + cb;
        *reinterpret_cast<float4*>(dst) = make_float4(o8[0], o8[1], o8[2], o8[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(o8[4], o8[5], o8[6], o8[7]);
    }
}

// ---------------------------------------------------------------------------
// scan: one 512-thread workgroup per (b, h, 64-column slice), both slices of a
// head on one XCD, chunks in order.  Its products run on the bf16 matrix cores
// with both factors split into bf16 hi + lo pairs (x = hi + lo to about 2^-18
// relative) and three products per pair: about 1e-5 relative per product,
// accumulated in fp32, the state carried in fp32.
//   Waves 0-3 (loaders) read each chunk's record, split it and write it to
// LDS as k32 operand fragments (16 rows x 32 k; lane (n, g) of the reader at
// entry n + 16 g holding row n with k = k0 + 4 g + e and k0 + 16 + 4 g + e):
// W and Q' (rows token, k channel), T and MT (rows token, k token; their six
// lower fragments), Kb^T (rows channel, k token) and gamma.  The first four
// and the last two are handed over separately, each in one buffer: the first
// four for chunk i + 1 are written while chunk i updates its state.
//   Waves 4-7 each keep a 128 x 16 fp32 slice of the state (value columns
// j0 .. j0 + 15) in registers as eight 16x16 accumulator tiles (rows 16 t +
// 4 g + e, column j0 + n), which in that k order are also the B operand of
// k32 block s = tiles 2 s, 2 s + 1; V comes straight from global memory a
// chunk ahead, and O goes straight out:
//   U = T V - W S,   O = scale (Q' S + MT V),   S <- Diag(gamma) S + Kb^T U.
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 512;
struct __align__(16) ScanLds {
    u32x4 wq[2][2][16 * b16::kFragLanes];  // [W, Q'][hi, lo][fragment 4 rt + s]
    u32x4 tm[2][2][6 * b16::kFragLanes];   // [T, MT][hi, lo][fragment: tri_rt, tri_s2]
    u32x4 kb[2][16 * b16::kFragLanes];     // [hi, lo][fragment 2 rt + s2]
    float gam[kD];
    // first part ready, first part consumed, Kb^T ready, Kb^T consumed (+4 a
    // chunk each; one buffer each, which keeps the roles in step), abort
    unsigned sync[5];
};

__global__ __launch_bounds__(kScanThreads, 1) void kda_chunk_scan_kernel(
    const uint8_t* __restrict__ ws, const float* __restrict__ v, const float* h_in,
    float* h_out, float* __restrict__ out, float scale, int T, int H, int chunk0, int nchunks,
    WaitCtl wait) {
    using R = RecF;
    using b16::frag_at;
    using b16::mma3;
    using b16::put_frag_hl;
    using b16::split_b;
    using b16::tri_rt;
    using b16::tri_s2;
    __shared__ ScanLds s;

    // Workgroups are dealt round-robin to the 8 XCDs (each with its own L2):
    // both slices of a head go to one XCD, so the records both read come from
    // HBM once.
    int slice, bh;
    {
        const int nblk = gridDim.x, id = blockIdx.x;
        const int per_xcd = nblk / 8;
        if (nblk % (8 * kScanSlices) == 0) {
            const int xcd = id % 8, idx = id / 8;
            bh = xcd * (per_xcd / kScanSlices) + idx / kScanSlices;
            slice = idx % kScanSlices;
        } else {
            slice = id % kScanSlices;
            bh = id / kScanSlices;
        }
    }
    const int h = bh % H, b = bh / H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;
    unsigned* const a_ready = &s.sync[0];
    unsigned* const a_done = &s.sync[1];
    unsigned* const k_ready = &s.sync[2];
    unsigned* const k_done = &s.sync[3];
    unsigned* const abort_w = &s.sync[4];
    if (tid < 5) s.sync[tid] = 0u;
    __syncthreads();  // the only workgroup barrier: roles split below

    if (wv < 4) {
        // ---- loaders: 16-byte pieces tid + 256 m of W, Q' (8 each), the
        // nonzero T and MT fragments (3 each), Kb^T (8) and gamma (threads < 32)
        float4 rw[8], rq[8], rt[3], rm[3], rk[8], rg = make_float4(0.f, 0.f, 0.f, 0.f);
        auto rec = [&](int cl) { return ws + ((size_t)bh * nchunks + cl) * R::BYTES; };
        auto issue_a = [&](int cl) {
            const float* Wg = reinterpret_cast<const float*>(rec(cl) + R::W);
            const float* Qg = reinterpret_cast<const float*>(rec(cl) + R::QP);
            const float* Tg = reinterpret_cast<const float*>(rec(cl) + R::TH);
            const float* Mg = reinterpret_cast<const float*>(rec(cl) + R::MH);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int p = tid + 256 * m, off = (p >> 5) * kD + 4 * (p & 31);
                rw[m] = *reinterpret_cast<const float4*>(Wg + off);
                rq[m] = *reinterpret_cast<const float4*>(Qg + off);
            }
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                const int p = tid + 256 * m, f = p >> 7, r16 = (p >> 3) & 15, q8 = p & 7;
                const int off = (16 * tri_rt(f) + r16) * kChunk + 32 * tri_s2(f) + 4 * q8;
                rt[m] = *reinterpret_cast<const float4*>(Tg + off);
                rm[m] = *reinterpret_cast<const float4*>(Mg + off);
            }
        };
        auto issue_k = [&](int cl) {
            const float* Kg = reinterpret_cast<const float*>(rec(cl) + R::KT);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int p = tid + 256 * m;
                rk[m] = *reinterpret_cast<const float4*>(Kg + (p >> 4) * kChunk + 4 * (p & 15));
            }
            if (tid < 32)
                rg = *reinterpret_cast<const float4*>(
                    reinterpret_cast<const float*>(rec(cl) + R::G) + 4 * tid);
        };
        issue_a(0);
        issue_k(0);
        for (int i = 0; i < nchunks; ++i) {
            // W, Q', T, MT once chunk i - 1 has multiplied them
            if (i >= 1) b16::wait_for(a_done, 4u * i, abort_w, wait.spin_limit);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int p = tid + 256 * m, ti = p >> 5, cq = p & 31;
                const int f = 4 * (ti >> 4) + (cq >> 3);
                put_frag_hl(s.wq[0][0], s.wq[0][1], f, ti & 15, cq & 3, (cq >> 2) & 1, rw[m]);
                put_frag_hl(s.wq[1][0], s.wq[1][1], f, ti & 15, cq & 3, (cq >> 2) & 1, rq[m]);
            }
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                const int p = tid + 256 * m, f = p >> 7, r16 = (p >> 3) & 15, q8 = p & 7;
                put_frag_hl(s.tm[0][0], s.tm[0][1], f, r16, q8 & 3, q8 >> 2, rt[m]);
                put_frag_hl(s.tm[1][0], s.tm[1][1], f, r16, q8 & 3, q8 >> 2, rm[m]);
            }
            b16::signal(a_ready, lane);
            if (i + 1 < nchunks) issue_a(i + 1);
            // Kb^T and gamma once chunk i - 1 has updated its state
            if (i >= 1) b16::wait_for(k_done, 4u * i, abort_w, wait.spin_limit);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int p = tid + 256 * m, ch = p >> 4, tq = p & 15;
                put_frag_hl(s.kb[0], s.kb[1], 2 * (ch >> 4) + (tq >> 3), ch & 15, tq & 3,
                            (tq >> 2) & 1, rk[m]);
            }
            if (tid < 32) *reinterpret_cast<float4*>(&s.gam[4 * tid]) = rg;
            b16::signal(k_ready, lane);
            if (i + 1 < nchunks) issue_k(i + 1);
        }
    } else {
        // ---- scan waves
        __builtin_amdgcn_s_setprio(3);
        const int j0 = kSliceCols * slice + 16 * (wv - 4);
        f32x4 S[8];
        const float* hin = h_in ? h_in + (size_t)bh * kD * kD : nullptr;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[t][e] = hin ? hin[(size_t)(16 * t + 4 * gq + e) * kD + j0 + n] : 0.f;
        // V at the lane's slots of a chunk (token 16 u + 4 gq + e, column j0 +
        // n; rows past the sequence read a valid row and are zeroed on use)
        float vr[16];
        const int64_t rstride = (int64_t)H * kD;
        const float* vbase = v + ((int64_t)b * T * H + h) * kD + j0 + n;
        auto vload = [&](int cl) {
            const int64_t t0 = (int64_t)(chunk0 + cl) * kChunk;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                int64_t tk = t0 + 16 * (m >> 2) + 4 * gq + (m & 3);
                tk = tk < T ? tk : T - 1;
                vr[m] = vbase[tk * rstride];
            }
        };
        vload(0);
        for (int i = 0; i < nchunks; ++i) {
            const int64_t t0 = (int64_t)(chunk0 + i) * kChunk;
            bf16x8 vh[2], vl[2];
            {
                f32x4 vt[4];
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    vt[m >> 2][m & 3] = t0 + 16 * (m >> 2) + 4 * gq + (m & 3) < T ? vr[m] : 0.f;
                split_b(vt[0], vt[1], vh[0], vl[0]);
                split_b(vt[2], vt[3], vh[1], vl[1]);
            }
            if (i + 1 < nchunks) vload(i + 1);
            bf16x8 sh[4], sl[4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) split_b(S[2 * sb], S[2 * sb + 1], sh[sb], sl[sb]);
            b16::wait_for(a_ready, 4u * (i + 1), abort_w, wait.spin_limit);
            // P = W S (rows 0..3) and Q' S (rows 4..7); TV and MT V
            f32x4 Pm[8], Tv[4], Mv[4];
#pragma unroll
            for (int r = 0; r < 8; ++r) Pm[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r) Tv[r] = Mv[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sb = 0; sb < 4; ++sb)
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt)
                        Pm[4 * x + rt] =
                            mma3(Pm[4 * x + rt], frag_at(s.wq[x][0], 4 * rt + sb, lane),
                                 frag_at(s.wq[x][1], 4 * rt + sb, lane), sh[sb], sl[sb]);
#pragma unroll
            for (int f = 0; f < 6; ++f) {
                Tv[tri_rt(f)] = mma3(Tv[tri_rt(f)], frag_at(s.tm[0][0], f, lane),
                                     frag_at(s.tm[0][1], f, lane), vh[tri_s2(f)], vl[tri_s2(f)]);
                Mv[tri_rt(f)] = mma3(Mv[tri_rt(f)], frag_at(s.tm[1][0], f, lane),
                                     frag_at(s.tm[1][1], f, lane), vh[tri_s2(f)], vl[tri_s2(f)]);
            }
            b16::signal(a_done, lane);
            // U = T V - W S as hi / lo; O = scale (Q' S + MT V)
            bf16x8 uh[2], ul[2];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) Tv[rt] -= Pm[rt];
            split_b(Tv[0], Tv[1], uh[0], ul[0]);
            split_b(Tv[2], Tv[3], uh[1], ul[1]);
            float* outc = out + ((int64_t)b * T * H + h) * kD + j0 + n;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const f32x4 o = scale * (Pm[4 + rt] + Mv[rt]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t tk = t0 + 16 * rt + 4 * gq + e;
                    if (tk < T) outc[tk * rstride] = o[e];
                }
            }
            // S <- Diag(gamma) S + Kb^T U
            b16::wait_for(k_ready, 4u * (i + 1), abort_w, wait.spin_limit);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                S[t] *= *reinterpret_cast<const f32x4*>(&s.gam[16 * t + 4 * gq]);
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    S[t] = mma3(S[t], frag_at(s.kb[0], 2 * t + s2, lane),
                                frag_at(s.kb[1], 2 * t + s2, lane), uh[s2], ul[s2]);
            }
            b16::signal(k_done, lane);
        }
        if (h_out) {
            float* ho = h_out + (size_t)bh * kD * kD;
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) ho[(size_t)(16 * t + 4 * gq + e) * kD + j0 + n] = S[t][e];
        }
    }
    // a wait of this wave (or of one that ended before) gave up: tell the host
    if (wait.abort_out && lane == 0 &&
        __hip_atomic_load(abort_w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0u)
        wait.abort_out[0] = 1u;
}

hipError_t launch_chunk_prep_f32(const float* q, const float* k, const float* g,
                                 const float* beta, int B, int T, int H, int chunk0, int nchunks,
                                 void* ws, hipStream_t stream, float* x_out) {
    const unsigned nblk = (unsigned)((int64_t)B * H * nchunks);
    hipLaunchKernelGGL(kda_chunk_prep_kernel<float>, dim3(nblk), dim3(256), 0, stream, q, k, g,
                       beta, T, H, chunk0, nchunks, static_cast<uint8_t*>(ws), x_out);
    return hipGetLastError();
}

hipError_t launch_chunk_prep_f32(const uint16_t* q, const uint16_t* k, const float* g,
                                 const float* beta, int B, int T, int H, int chunk0, int nchunks,
                                 void* ws, hipStream_t stream, float* x_out) {
    const unsigned nblk = (unsigned)((int64_t)B * H * nchunks);
    hipLaunchKernelGGL(kda_chunk_prep_kernel<uint16_t>, dim3(nblk), dim3(256), 0, stream, q, k,
                       g, beta, T, H, chunk0, nchunks, static_cast<uint8_t*>(ws), x_out);
    return hipGetLastError();
}

hipError_t launch_chunk_scan_f32(const void* ws, const float* v, const float* h_in, float* h_out,
                                 float* out, float scale, int B, int T, int H, int chunk0,
                                 int nchunks, const WaitCtl& wait, hipStream_t stream) {
    const unsigned nblk = (unsigned)((int64_t)B * H * kScanSlices);
    hipLaunchKernelGGL(kda_chunk_scan_kernel, dim3(nblk), dim3(kScanThreads), 0, stream,
                       static_cast<const uint8_t*>(ws), v, h_in, h_out, out, scale, T, H, chunk0,
                       nchunks, wait);
    return hipGetLastError();
}

}  // namespace kda
