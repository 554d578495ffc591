// Backward of the chunkwise prefill, for fp32 or bf16 q / k / v / dout (and
// dq / dk / dv in the same type; all arithmetic fp32): the gradients of
// L = <dO, O> + <dS_T, S_T> with respect to q, k, v, g, beta and the initial
// state, for O, S_T computed by the Kimi Delta Attention recurrence (Kimi-K3
// 深度解析 blog, section 三; the KDA paragraph of the 深入 Kimi-K3 thread for
// the in-kernel L2 normalisation and the per-channel decay).  The pages give
// no backward; this is the reverse-mode derivative of the chunk form written
// out in kda_chunk.hip.
//
// Per 64-token chunk entering with state S and leaving with S', with R = V -
// Kt S, U = T R and the quantities of the chunk form (Kt, Qt, Kb, gamma, the
// pairwise-decayed products P = strict-lower(kh kh^T decayed) and N =
// lower-incl(qh kh^T decayed), A = diag(beta) P, X = (I + A)^-1, T = X
// diag(beta), M = N), the gradients given dO and dS' = dL/dS' are
//   dU  = scale M^T dO + Kb dS'          dV = dR = T^T dU
//   dS  = Diag(gamma) dS' - W^T (Kb dS') + scale Q'^T dO      (W = T Kt,
//                                                   Q' = Qt - M W)
//   dT  = lower-incl(dU R^T),  dX = dT diag(beta),  dbeta_i += sum_r X_ri dT_ri
//   dA  = -strict-lower(X^T dX X^T), dbeta_r += sum_i dA_ri P_ri, dP = diag(beta) dA
//   dM  = scale lower-incl(dO U^T)
//   dQt = scale dO S^T,  dKt = -dR S^T,  dKb = U dS'^T,  dgamma = rowsum(dS' . S)
// then through the decay factors into dkh, dqh and the in-chunk cumulative
// log-decay Gam (whose reverse cumulative sum is dg), and through the L2
// normalisation into dq, dk.  dS depends on dS' and dO column by column, as S'
// on S in the forward, so it runs as a scan over chunks in reverse; all other
// gradients of a chunk follow from S and dS' alone, in parallel over chunks.
//
// Four launches:
//   prep  (kda_chunk.hip) writes each chunk's record (W, Q', Kb^T, T and
//         gamma; no M T, which only the forward scan reads), X = (I + A)^-1,
//         P = strict-lower(KK) and N = M;
//   state scan    walks the chunks forward and stores the state entering each;
//   gradient scan walks them in reverse and stores dS' of each chunk, and dS
//         of the first as the initial state's gradient;
//   chunk gradients, one workgroup per (batch, head, chunk), rebuilds the
//         decay factors and the chunk's [64][128] matrices from q, k, g, beta,
//         takes X, P and N from prep, and writes dq, dk, dv, dg, dbeta.
// Every product runs on the matrix cores with its operands in LDS or
// registers: the scans' products and the chunk kernel's [64][128] ones as
// three bf16 products per hi / lo pair, the chunk kernel's [64][64] ones in
// fp32 (v_mfma_f32_16x16x4_f32).
#include "kda_bf16.hpp"
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace {

using RF = ChunkRecF32;
constexpr int kScanCols = 64;              // value columns per scan workgroup
constexpr int kScanSlices = kD / kScanCols;
constexpr int kScanThreads = 512;
constexpr size_t kStateFloats = (size_t)kD * kD;


__device__ __forceinline__ float ex(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ float4 ld4(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
// dq / dk / dv out: fp32, or bf16 rounded to nearest even
__device__ __forceinline__ void io_st(float* p, float x) { *p = x; }
__device__ __forceinline__ void io_st(uint16_t* p, float x) { *p = f2bf(x); }

__device__ __forceinline__ float4 mul4(float4 a, float4 b) {
    return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}
__device__ __forceinline__ float4 exp4(float4 a) {
    return make_float4(ex(a.x), ex(a.y), ex(a.z), ex(a.w));
}
__device__ __forceinline__ float4 scale4(float4 a, float c) {
    return make_float4(a.x * c, a.y * c, a.z * c, a.w * c);
}

__device__ __forceinline__ void scan_ids(int& bh, int& slice) {
    // all slices of one head on one XCD (workgroups are dealt round-robin to
    // the 8 XCDs), so the records they share come from HBM once
    const int nb = gridDim.x;
    const int id = blockIdx.x;
    if (nb % (8 * kScanSlices) == 0) {
        const int xcd = id % 8, j = id / 8;
        const int per = nb / 8;  // workgroups per XCD, a multiple of kScanSlices
        const int w = xcd * per + j;
        bh = w / kScanSlices;
        slice = w % kScanSlices;
    } else {
        bh = id / kScanSlices;
        slice = id % kScanSlices;
    }
}

// ---------------------------------------------------------------------------
// The two scans: one 512-thread workgroup per (b, h, 64 value columns), both
// slices of a head on one XCD.  Their products run on the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16) with every operand split into a bf16 pair, x =
// hi + lo to about 2^-18 relative, and three products per pair (hi hi + hi lo
// + lo hi): about 1e-5 relative per product, accumulated in fp32, with the
// state (or its gradient) carried in fp32.
//   Waves 0-3 (loaders) read each chunk's record from global memory, split it
// and write it to LDS as k32 operand fragments: 16 rows x 32 k, 1 KB of hi
// and 1 KB of lo, lane (n, g) of the reading wave at byte 16 (n + 16 g)
// holding row n with k = k0 + 4 g + e (values 0..3) and k0 + 16 + 4 g + e
// (values 4..7).  A matrix the products need with its other index as rows is
// read column-wise from the record (64 consecutive floats per load across the
// wave), so no transposition pass is needed.
//   Waves 4-7 each keep a 128 x 16 fp32 slice (value columns j0 .. j0 + 15) in
// registers as eight 16x16 accumulator tiles (rows 16 t + 4 g + e, column
// j0 + n).  In that k order the tiles 2 s and 2 s + 1 are the B operand of
// k32 block s, so the state and every product result feed the next product
// from registers; V and dO come straight from global memory, a chunk ahead.
//   The roles hand the fragments over through LDS counters, never through a
// workgroup barrier.
// ---------------------------------------------------------------------------

using b16::mma;
using b16::signal;
using b16::split_b;
using b16::wait_for;
using b16::kFragLanes;
using b16::mma3;
using b16::tri_rt;
using b16::tri_s2;

// Raw q / k / v / dout values, held in registers until they are used (widening
// a bf16 value is an instruction, which would make the wave wait for the load
// where it is placed).
template <typename IO> struct RawIO;
template <> struct RawIO<float> {
    using one = float;
    using four = float4;
    static __device__ __forceinline__ float wid(float x) { return x; }
    static __device__ __forceinline__ float4 wid(float4 x) { return x; }
};
template <> struct RawIO<uint16_t> {
    using one = uint16_t;
    using four = uint2;
    static __device__ __forceinline__ float wid(uint16_t x) { return bf2f(x); }
    static __device__ __forceinline__ float4 wid(uint2 u) {
        return make_float4(__builtin_bit_cast(float, u.x << 16),
                           __builtin_bit_cast(float, u.x & 0xffff0000u),
                           __builtin_bit_cast(float, u.y << 16),
                           __builtin_bit_cast(float, u.y & 0xffff0000u));
    }
};

// ---------------------------------------------------------------------------
// State scan: chunks in order.  For chunk c the state slice entering it is
// stored, then Z = T V - W S and S <- Diag(gamma) S + Kb^T Z.  Each chunk's
// fragments (W: rows token, k channel; T: rows token, k token; Kb^T: rows
// channel, k token) and gamma sit in two LDS buffers by chunk parity, so the
// loaders fill chunk i + 1 while chunk i is scanned.
// ---------------------------------------------------------------------------
struct __align__(16) StateScanLds {
    u32x4 w[2][2][16 * kFragLanes];   // [buffer][hi, lo][fragment 4 rt + s]
    u32x4 t[2][2][6 * kFragLanes];    // [buffer][hi, lo][fragment: tri_rt, tri_s2]
    u32x4 kb[2][2][16 * kFragLanes];  // [buffer][hi, lo][fragment 2 rt + s2]
    float gam[2][kD];
    // per buffer: its chunks ready, its chunks consumed (+4 each); abort.  One
    // counter per buffer: waves of a role may be a chunk apart, and a shared
    // counter would let the later chunk's signals stand in for the earlier's.
    unsigned sync[5];
};

// Chunks chunk0 .. chunk0 + nch - 1 of the sequence (records, states local to
// the segment); h_out (or NULL) receives the state leaving the last one.
template <typename IO>
__global__ __launch_bounds__(kScanThreads, 1) void kda_bwd_state_scan_kernel(
    const uint8_t* __restrict__ rec, const IO* __restrict__ v, const float* __restrict__ h0,
    float* __restrict__ states, float* __restrict__ h_out, int T, int H, int chunk0, int nch,
    WaitCtl wait) {
    using RW = RawIO<IO>;
    __shared__ StateScanLds s;
    int bh, slice;
    scan_ids(bh, slice);
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;
    unsigned* const ready = &s.sync[0];     // [buffer]
    unsigned* const consumed = &s.sync[2];  // [buffer]
    unsigned* const abort_w = &s.sync[4];
    if (tid < 5) s.sync[tid] = 0u;
    __syncthreads();  // the only workgroup barrier: roles split below

    if (wv < 4) {
        // ---- loaders: 16-byte pieces tid + 256 m of W (8), Kb^T (8), the
        // nonzero T fragments (3) and gamma (threads < 32), a chunk ahead
        static_assert(kScanThreads == 512, "four loader waves");
        float4 rw[8], rk[8], rt[3], rg = make_float4(0.f, 0.f, 0.f, 0.f);
        auto issue = [&](int c) {
            const uint8_t* r = rec + ((size_t)bh * nch + c) * RF::BYTES;
            const float* Wg = reinterpret_cast<const float*>(r + RF::W);
            const float* Kg = reinterpret_cast<const float*>(r + RF::KT);
            const float* Tg = reinterpret_cast<const float*>(r + RF::TH);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int p = tid + 256 * m;
                rw[m] = ld4(Wg + (p >> 5) * kD + 4 * (p & 31));
                rk[m] = ld4(Kg + (p >> 4) * kChunk + 4 * (p & 15));
            }
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                const int p = tid + 256 * m, f = p >> 7, r16 = (p >> 3) & 15, q8 = p & 7;
                rt[m] = ld4(Tg + (16 * tri_rt(f) + r16) * kChunk + 32 * tri_s2(f) + 4 * q8);
            }
            if (tid < 32) rg = ld4(reinterpret_cast<const float*>(r + RF::G) + 4 * tid);
        };
        auto put = [&](int bf) {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int p = tid + 256 * m;
                {  // W: token i = p / 32, channels 4 cq ..
                    const int i = p >> 5, cq = p & 31;
                    b16::put_frag_hl(s.w[bf][0], s.w[bf][1], 4 * (i >> 4) + (cq >> 3), i & 15, cq & 3,
                             (cq >> 2) & 1, rw[m]);
                }
                {  // Kb^T: channel ch = p / 16, tokens 4 tq ..
                    const int ch = p >> 4, tq = p & 15;
                    b16::put_frag_hl(s.kb[bf][0], s.kb[bf][1], 2 * (ch >> 4) + (tq >> 3), ch & 15, tq & 3,
                             (tq >> 2) & 1, rk[m]);
                }
            }
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                const int p = tid + 256 * m, f = p >> 7, r16 = (p >> 3) & 15, q8 = p & 7;
                b16::put_frag_hl(s.t[bf][0], s.t[bf][1], f, r16, q8 & 3, q8 >> 2, rt[m]);
            }
            if (tid < 32) *reinterpret_cast<float4*>(&s.gam[bf][4 * tid]) = rg;
        };
        // chunk i into buffer i & 1, free once chunk i - 2 (the buffer's
        // previous chunk, its round i / 2 - 1) is consumed
        issue(0);
        for (int i = 0; i < nch; ++i) {
            const int bf = i & 1;
            wait_for(&consumed[bf], 4u * (unsigned)(i >> 1), abort_w, wait.spin_limit);
            put(bf);
            signal(&ready[bf], lane);
            if (i + 1 < nch) issue(i + 1);
        }
    } else {
        // ---- scan waves
        __builtin_amdgcn_s_setprio(3);
        const int j0 = kScanCols * slice + 16 * (wv - 4);
        f32x4 S[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[t][e] = h0 ? h0[(size_t)bh * kStateFloats + (size_t)(16 * t + 4 * gq + e) * kD + j0 + n]
                             : 0.f;
        // V at the lane's slots of a chunk (token 16 u + 4 gq + e, column j0 +
        // n; rows past the sequence read a valid row and are zeroed on use)
        typename RW::one vr[16];
        auto vload = [&](int c) {
            const int64_t t0 = (int64_t)(chunk0 + c) * kChunk;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                int64_t tk = t0 + 16 * (m >> 2) + 4 * gq + (m & 3);
                tk = tk < T ? tk : T - 1;
                vr[m] = v[(((int64_t)b * T + tk) * H + h) * kD + j0 + n];
            }
        };
        vload(0);
        for (int i = 0; i < nch; ++i) {
            const int bf = i & 1;
            const int64_t t0 = (int64_t)(chunk0 + i) * kChunk;
            // V as hi / lo B operands (k32 block s2 = tiles 2 s2, 2 s2 + 1)
            bf16x8 vh[2], vl[2];
            {
                f32x4 vt[4];
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    vt[m >> 2][m & 3] =
                        t0 + 16 * (m >> 2) + 4 * gq + (m & 3) < T ? RW::wid(vr[m]) : 0.f;
                split_b(vt[0], vt[1], vh[0], vl[0]);
                split_b(vt[2], vt[3], vh[1], vl[1]);
            }
            if (i + 1 < nch) vload(i + 1);
            float* st = states + ((size_t)bh * nch + i) * kStateFloats;
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) st[(size_t)(16 * t + 4 * gq + e) * kD + j0 + n] = S[t][e];
            bf16x8 sh[4], sl[4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) split_b(S[2 * sb], S[2 * sb + 1], sh[sb], sl[sb]);
            wait_for(&ready[bf], 4u * ((i >> 1) + 1), abort_w, wait.spin_limit);
            // Z = T V - W S  (T lower triangular: six fragments)
            f32x4 Z[4], P[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) Z[rt] = P[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sb = 0; sb < 4; ++sb)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
                    P[rt] = mma3(P[rt], b16::frag_at(s.w[bf][0], 4 * rt + sb, lane),
                                 b16::frag_at(s.w[bf][1], 4 * rt + sb, lane), sh[sb], sl[sb]);
#pragma unroll
            for (int f = 0; f < 6; ++f)
                Z[tri_rt(f)] = mma3(Z[tri_rt(f)], b16::frag_at(s.t[bf][0], f, lane),
                                    b16::frag_at(s.t[bf][1], f, lane), vh[tri_s2(f)], vl[tri_s2(f)]);
            bf16x8 zh[2], zl[2];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) Z[rt] -= P[rt];
            split_b(Z[0], Z[1], zh[0], zl[0]);
            split_b(Z[2], Z[3], zh[1], zl[1]);
            // S <- Diag(gamma) S + Kb^T Z
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                S[t] *= *reinterpret_cast<const f32x4*>(&s.gam[bf][16 * t + 4 * gq]);
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    S[t] = mma3(S[t], b16::frag_at(s.kb[bf][0], 2 * t + s2, lane),
                                b16::frag_at(s.kb[bf][1], 2 * t + s2, lane), zh[s2], zl[s2]);
            }
            signal(&consumed[bf], lane);
        }
        if (h_out) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    h_out[(size_t)bh * kStateFloats + (size_t)(16 * t + 4 * gq + e) * kD + j0 + n] =
                        S[t][e];
        }
    }
    // a wait of this wave (or of one that ended before) gave up: tell the host
    if (wait.abort_out && lane == 0 &&
        __hip_atomic_load(abort_w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0u)
        wait.abort_out[0] = 1u;
}

// ---------------------------------------------------------------------------
// Gradient scan: chunks in reverse.  For chunk c, dS' (the gradient of the
// state leaving it) is stored, then Y = Kb dS' and
//   dS <- Diag(gamma) dS' - W^T Y + scale Q'^T dO.
// After chunk 0, dS is the initial state's gradient.  The Kb fragments (rows
// token, k channel; read column-wise from the Kb^T record) sit in two buffers
// by chunk parity; -W^T and scale Q'^T (rows channel, k token; read
// column-wise from the W and Q' records, sign and scale applied before the
// split) and gamma in one, refilled while the next chunk forms Y.
// ---------------------------------------------------------------------------
struct __align__(16) GradScanLds {
    u32x4 kb[2][2][16 * kFragLanes];  // [buffer][hi, lo][fragment 4 rt + s]
    u32x4 wq[2][2][16 * kFragLanes];  // [-W^T, scale Q'^T][hi, lo][fragment 2 rt + s2]
    float gam[kD];
    // Kb ready and Kb consumed per buffer, W / Q ready, W / Q consumed (+4 a
    // chunk each), abort.  The double-buffered Kb needs a counter per buffer
    // (waves of a role may be a chunk apart); the single W / Q buffer keeps
    // the roles in step by itself.
    unsigned sync[7];
};

// Chunks chunk0 .. chunk0 + nch - 1 (records and dS' local to the segment):
// dhT is the gradient of the state leaving the last of them, dh0 receives that
// of the state entering the first.  dh0 may equal dhT (each workgroup reads its
// slice before it writes it).
template <typename IO>
__global__ __launch_bounds__(kScanThreads, 1) void kda_bwd_grad_scan_kernel(
    const uint8_t* __restrict__ rec, const IO* __restrict__ dout, const float* dhT,
    float* __restrict__ dsn, float* dh0, float scale, int T, int H, int chunk0, int nch,
    WaitCtl wait) {
    using RW = RawIO<IO>;
    __shared__ GradScanLds s;
    int bh, slice;
    scan_ids(bh, slice);
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;
    unsigned* const kb_ready = &s.sync[0];  // [buffer]
    unsigned* const kb_done = &s.sync[2];   // [buffer]
    unsigned* const wq_ready = &s.sync[4];
    unsigned* const wq_done = &s.sync[5];
    unsigned* const abort_w = &s.sync[6];
    if (tid < 7) s.sync[tid] = 0u;
    __syncthreads();  // the only workgroup barrier: roles split below

    if (wv < 4) {
        // ---- loaders: piece tid + 256 m (m < 8) of Kb (token p % 64, channels
        // 4 (p / 64) ..) and of -W^T, scale Q'^T (channel p % 128, tokens
        // 4 (p / 128) ..), four column-wise loads each; gamma (threads < 32)
        float4 rk[8], rw[8], rq[8], rg = make_float4(0.f, 0.f, 0.f, 0.f);
        auto issue_kb = [&](int c) {
            const float* Kg = reinterpret_cast<const float*>(
                rec + ((size_t)bh * nch + c) * RF::BYTES + RF::KT);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int p = tid + 256 * m, i = p & 63, c0 = 4 * (p >> 6);
                rk[m] = make_float4(Kg[(c0 + 0) * kChunk + i], Kg[(c0 + 1) * kChunk + i],
                                    Kg[(c0 + 2) * kChunk + i], Kg[(c0 + 3) * kChunk + i]);
            }
        };
        auto issue_wq = [&](int c) {
            const uint8_t* r = rec + ((size_t)bh * nch + c) * RF::BYTES;
            const float* Wg = reinterpret_cast<const float*>(r + RF::W);
            const float* Qg = reinterpret_cast<const float*>(r + RF::QP);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int p = tid + 256 * m, ch = p & 127, t0 = 4 * (p >> 7);
                rw[m] = make_float4(Wg[(t0 + 0) * kD + ch], Wg[(t0 + 1) * kD + ch],
                                    Wg[(t0 + 2) * kD + ch], Wg[(t0 + 3) * kD + ch]);
                rq[m] = make_float4(Qg[(t0 + 0) * kD + ch], Qg[(t0 + 1) * kD + ch],
                                    Qg[(t0 + 2) * kD + ch], Qg[(t0 + 3) * kD + ch]);
            }
            if (tid < 32) rg = ld4(reinterpret_cast<const float*>(r + RF::G) + 4 * tid);
        };
        // chunk i (sequence chunk nch - 1 - i): Kb into buffer i & 1 once chunk
        // i - 2 (the buffer's previous one) has formed its Y; -W^T, scale Q'^T
        // and gamma once chunk i - 1 is done with them
        issue_kb(nch - 1);
        issue_wq(nch - 1);
        for (int i = 0; i < nch; ++i) {
            const int c = nch - 1 - i, bf = i & 1;
            wait_for(&kb_done[bf], 4u * (unsigned)(i >> 1), abort_w, wait.spin_limit);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int p = tid + 256 * m, ti = p & 63, cq = p >> 6;
                b16::put_frag_hl(s.kb[bf][0], s.kb[bf][1], 4 * (ti >> 4) + (cq >> 3), ti & 15, cq & 3,
                         (cq >> 2) & 1, rk[m]);
            }
            signal(&kb_ready[bf], lane);
            if (c > 0) issue_kb(c - 1);
            if (i >= 1) wait_for(wq_done, 4u * i, abort_w, wait.spin_limit);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int p = tid + 256 * m, ch = p & 127, tq = p >> 7;
                const int f = 2 * (ch >> 4) + (tq >> 3);
                b16::put_frag_hl(s.wq[0][0], s.wq[0][1], f, ch & 15, tq & 3, (tq >> 2) & 1,
                         scale4(rw[m], -1.f));
                b16::put_frag_hl(s.wq[1][0], s.wq[1][1], f, ch & 15, tq & 3, (tq >> 2) & 1,
                         scale4(rq[m], scale));
            }
            if (tid < 32) *reinterpret_cast<float4*>(&s.gam[4 * tid]) = rg;
            signal(wq_ready, lane);
            if (c > 0) issue_wq(c - 1);
        }
    } else {
        // ---- scan waves
        __builtin_amdgcn_s_setprio(3);
        const int j0 = kScanCols * slice + 16 * (wv - 4);
        f32x4 D[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                D[t][e] = dhT ? dhT[(size_t)bh * kStateFloats + (size_t)(16 * t + 4 * gq + e) * kD + j0 + n]
                              : 0.f;
        typename RW::one orw[16];
        auto oload = [&](int c) {
            const int64_t t0 = (int64_t)(chunk0 + c) * kChunk;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                int64_t tk = t0 + 16 * (m >> 2) + 4 * gq + (m & 3);
                tk = tk < T ? tk : T - 1;
                orw[m] = dout[(((int64_t)b * T + tk) * H + h) * kD + j0 + n];
            }
        };
        oload(nch - 1);
        for (int i = 0; i < nch; ++i) {
            const int c = nch - 1 - i, bf = i & 1;
            const int64_t t0 = (int64_t)(chunk0 + c) * kChunk;
            bf16x8 oh[2], ol[2];
            {
                f32x4 ot[4];
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    ot[m >> 2][m & 3] =
                        t0 + 16 * (m >> 2) + 4 * gq + (m & 3) < T ? RW::wid(orw[m]) : 0.f;
                split_b(ot[0], ot[1], oh[0], ol[0]);
                split_b(ot[2], ot[3], oh[1], ol[1]);
            }
            if (c > 0) oload(c - 1);
            float* st = dsn + ((size_t)bh * nch + c) * kStateFloats;
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) st[(size_t)(16 * t + 4 * gq + e) * kD + j0 + n] = D[t][e];
            bf16x8 dh[4], dl[4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) split_b(D[2 * sb], D[2 * sb + 1], dh[sb], dl[sb]);
            // Y = Kb dS'
            wait_for(&kb_ready[bf], 4u * ((i >> 1) + 1), abort_w, wait.spin_limit);
            f32x4 Y[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) Y[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sb = 0; sb < 4; ++sb)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
                    Y[rt] = mma3(Y[rt], b16::frag_at(s.kb[bf][0], 4 * rt + sb, lane),
                                 b16::frag_at(s.kb[bf][1], 4 * rt + sb, lane), dh[sb], dl[sb]);
            signal(&kb_done[bf], lane);
            bf16x8 yh[2], yl[2];
            split_b(Y[0], Y[1], yh[0], yl[0]);
            split_b(Y[2], Y[3], yh[1], yl[1]);
            // dS = Diag(gamma) dS' - W^T Y + scale Q'^T dO
            wait_for(wq_ready, 4u * (i + 1), abort_w, wait.spin_limit);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                D[t] *= *reinterpret_cast<const f32x4*>(&s.gam[16 * t + 4 * gq]);
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    D[t] = mma3(D[t], b16::frag_at(s.wq[0][0], 2 * t + s2, lane),
                                b16::frag_at(s.wq[0][1], 2 * t + s2, lane), yh[s2], yl[s2]);
                    D[t] = mma3(D[t], b16::frag_at(s.wq[1][0], 2 * t + s2, lane),
                                b16::frag_at(s.wq[1][1], 2 * t + s2, lane), oh[s2], ol[s2]);
                }
            }
            signal(wq_done, lane);
        }
        if (dh0) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dh0[(size_t)bh * kStateFloats + (size_t)(16 * t + 4 * gq + e) * kD + j0 + n] =
                        D[t][e];
        }
    }
    if (wait.abort_out && lane == 0 &&
        __hip_atomic_load(abort_w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0u)
        wait.abort_out[0] = 1u;
}

// ---------------------------------------------------------------------------
// Chunk gradients: one 512-thread workgroup per (b, h, chunk), two waves per
// SIMD; every intermediate stays in registers or LDS.
//
// Lane (n, gq) of wave w owns channel cc = 16 w + n of the rows 16 u + 4 gq + e
// (u, e < 4; slot m = 4 u + e): the accumulator layout of column tile w of a
// 64 x 128 product in which wave w computes all four row tiles.  A 16-token
// block kb of a contraction over tokens takes its B operand straight from the
// owned slots 4 kb .. 4 kb + 3 of a [64][128] result, so U = T R and dR =
// T^T dU run from registers.  The products that contract over channels read
// their operands as 16-byte rows from LDS, where each such result is staged
// once.  The B operands that come from the state and its gradient (a wave's
// 16 columns, or its 16 rows, of S and dS') are loaded into registers one
// phase before they are used.
//
// LDS: three [64][132] arrays (kh, qh and Gam, then
// Kt and Kb for R and dU, then R, dU and U, then scale dO, dX / Y and dR), P,
// N and X at a pitch of 68 (16-byte rows that a wave reads in 8 distinct bank
// groups), and a few vectors.  Partial sums are reduced in a fixed order, so
// results are bitwise reproducible.
// ---------------------------------------------------------------------------
constexpr int kCT = 512;
constexpr int kPB = kD + 4;      // pitch of the [64][128] arrays
constexpr int kPS = kChunk + 4;  // pitch of the [64][64] arrays
struct __align__(16) BwdLds {
    float big[3][kChunk][kPB];
    float p[kChunk][kPS];  // P, later dP
    float n[kChunk][kPS];  // N (= M), later dM
    float x[kChunk][kPS];  // X = (I + A)^-1
    float beta[kChunk];
    float rq[kChunk];
    float rk[kChunk];
    float dbeta[kChunk];
    float dotq[kChunk];
    float dotk[kChunk];
    float gl[kD];     // Gam of the chunk's last row
    float red[8 * kD];  // partial sums
};
static_assert(kPS <= kPB, "dX, then Y, fit in one [64][128] array");

// The lane's 16 owned values of a [64][128] matrix (slot m: row 16 (m / 4) +
// 4 gq + m % 4, channel 16 wv + n) into its hi / lo k32 fragments (rows token,
// k channel; fragment 4 (row / 16) + channel / 32), one bf16 of each per value.
__device__ __forceinline__ void stage_own(u32x4* hi, u32x4* lo, const float (&x)[16], int wv,
                                          int n, int gq) {
    uint16_t* h16 = reinterpret_cast<uint16_t*>(hi);
    uint16_t* l16 = reinterpret_cast<uint16_t*>(lo);
    // within fragment wv / 2: lane slot (row % 16, (n / 4)), half wv % 2, value n % 4
    const int base = 8 * (b16::kFragLanes * (wv >> 1) + 16 * (n >> 2)) + 4 * (wv & 1) + (n & 3);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int idx = base + 8 * (b16::kFragLanes * 4 * (m >> 2) + 4 * gq + (m & 3));
        const __bf16 hb = (__bf16)x[m];
        const __bf16 lb = (__bf16)(x[m] - (float)hb);
        h16[idx] = __builtin_bit_cast(uint16_t, hb);
        l16[idx] = __builtin_bit_cast(uint16_t, lb);
    }
}

// acc += A B over one 4-deep step per component: four fp32 MFMAs
__device__ __forceinline__ void mfma4(f32x4& acc, float4 a, float4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
}

// Sums each of V values (V a power of two) over the 16 lanes n of a row by
// halving exchanges.  On return x[j] of lane n holds the sum of value
// (V / 16) n + j (j < V / 16) for V >= 16, or of value n / (16 / V) for V < 16.
template <int LEN, int MASK, int V>
__device__ __forceinline__ void rsum_step(float (&x)[V], int n) {
    if constexpr (MASK >= 1) {
        if constexpr (LEN > 1) {
            constexpr int HALF = LEN / 2;
            const bool hi = (n & MASK) != 0;
#pragma unroll
            for (int i = 0; i < HALF; ++i) {
                const float keep = hi ? x[HALF + i] : x[i];
                const float send = hi ? x[i] : x[HALF + i];
                x[i] = keep + __shfl_xor(send, MASK);
            }
            rsum_step<HALF, MASK / 2>(x, n);
        } else {
            x[0] += __shfl_xor(x[0], MASK);
            rsum_step<1, MASK / 2>(x, n);
        }
    }
}
template <int V>
__device__ __forceinline__ void row_sums(float (&x)[V], int n) {
    rsum_step<V, 8>(x, n);
}

template <typename IO>
__global__ __launch_bounds__(kCT, 1) void kda_bwd_chunk_kernel(
    const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const IO* __restrict__ dout,
    const float* __restrict__ states, const float* __restrict__ dsn,
    const float* __restrict__ xs, float scale, int T, int H, int chunk0, int nch,
    IO* __restrict__ dq, IO* __restrict__ dk, IO* __restrict__ dv, float* __restrict__ dg,
    float* __restrict__ dbeta) {
    using RW = RawIO<IO>;
    __shared__ BwdLds s;
    // fp32 rows: kh, qh and Gam
    float(*const A0)[kPB] = s.big[0];
    float(*const A1)[kPB] = s.big[1];
    float(*const A2)[kPB] = s.big[2];
    // then the same space as bf16 hi / lo k32 fragments (rows token, k channel):
    // F0: -Kt, R, dR;  F1: Kb, dU, scale dO;  F2: U
    auto fh = [&](int k) { return reinterpret_cast<u32x4*>(&s.big[k][0][0]); };
    auto fl = [&](int k) { return reinterpret_cast<u32x4*>(&s.big[k][0][0]) + 16 * b16::kFragLanes; };
    float(*const DX)[kPS] = reinterpret_cast<float(*)[kPS]>(&s.big[0][0][0]);  // dX, then Y

    // chunk c of the segment (states, dS', X) is chunk cg of the sequence
    const int c = blockIdx.x % nch;
    const int bh = blockIdx.x / nch;
    const int b = bh / H, h = bh % H;
    const int cg = chunk0 + c;
    const int L = min(kChunk, T - cg * kChunk);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;
    const int cc = 16 * wv + n;
    const size_t rp = (size_t)H * kD;  // pitch of one token row
    const size_t base = (((size_t)b * T + (size_t)cg * kChunk) * H + h) * kD;
    const float* S = states + (size_t)blockIdx.x * kStateFloats;
    const float* dSn = dsn + (size_t)blockIdx.x * kStateFloats;
    // row of owned slot m; rows past the sequence read row L - 1 and are zeroed on use
    auto orow = [&](int m) { return 16 * (m >> 2) + 4 * gq + (m & 3); };
    auto crow = [&](int r) { return min(r, L - 1); };

    // ---- loads: q, k, g (8 threads per row, 16 channels each), X, P and N
    // (into LDS at once), then the column strips of S and dS' (B operands of R
    // and dU), v and dout
    float scol[32], dcol[32];  // S, dS' at [16 kb + 4 gq + e][cc], slot 4 kb + e
    typename RW::one vraw[16], oraw[16];
    float4 xpf[2], pnf[4];
    {
        const int r = tid >> 3, part = tid & 7;
        typename RW::four qr[4], kr[4];
        float4 gv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t off = base + (size_t)crow(r) * rp + 16 * part + 4 * e;
            qr[e] = *reinterpret_cast<const typename RW::four*>(q + off);
            kr[e] = *reinterpret_cast<const typename RW::four*>(k + off);
            gv[e] = ld4(g + off);
        }
        const float bt = beta[((size_t)b * T + (size_t)cg * kChunk + crow(r)) * H + h];
        const float* Xg = xs + (size_t)blockIdx.x * 3 * kChunk * kChunk;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = tid + kCT * j;
            xpf[j] = ld4(Xg + (e >> 4) * kChunk + 4 * (e & 15));
            pnf[j] = ld4(Xg + kChunk * kChunk + (e >> 4) * kChunk + 4 * (e & 15));
            pnf[2 + j] = ld4(Xg + 2 * kChunk * kChunk + (e >> 4) * kChunk + 4 * (e & 15));
        }
#pragma unroll
        for (int t = 0; t < 32; ++t)
            scol[t] = S[(size_t)(16 * (t >> 2) + 4 * gq + (t & 3)) * kD + cc];
        __builtin_amdgcn_sched_barrier(0);
        const bool ok = r < L;
        float4 qv[4], kv[4];
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qv[e] = RW::wid(qr[e]);
            kv[e] = RW::wid(kr[e]);
            sq += qv[e].x * qv[e].x + qv[e].y * qv[e].y + qv[e].z * qv[e].z + qv[e].w * qv[e].w;
            sk += kv[e].x * kv[e].x + kv[e].y * kv[e].y + kv[e].z * kv[e].z + kv[e].w * kv[e].w;
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) {
            sq += __shfl_xor(sq, o);
            sk += __shfl_xor(sk, o);
        }
        // rows past the sequence: qh = kh = 0 and g = 0 (Gam stays at its last value)
        const float rq = ok ? 1.f / sqrtf(sq + kNormEps) : 0.f;
        const float rk = ok ? 1.f / sqrtf(sk + kNormEps) : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int col = 16 * part + 4 * e;
            *reinterpret_cast<float4*>(&A0[r][col]) = scale4(kv[e], rk);
            *reinterpret_cast<float4*>(&A1[r][col]) = scale4(qv[e], rq);
            *reinterpret_cast<float4*>(&A2[r][col]) = ok ? gv[e] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (part == 0) {
            s.rq[r] = rq;
            s.rk[r] = rk;
            s.beta[r] = ok ? bt : 0.f;
        }
        // X, P and N as prep wrote them (P and N zero above their diagonal blocks)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = tid + kCT * j;
            *reinterpret_cast<float4*>(&s.x[e >> 4][4 * (e & 15)]) = xpf[j];
            *reinterpret_cast<float4*>(&s.p[e >> 4][4 * (e & 15)]) = pnf[j];
            *reinterpret_cast<float4*>(&s.n[e >> 4][4 * (e & 15)]) = pnf[2 + j];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 32; ++t)
            dcol[t] = dSn[(size_t)(16 * (t >> 2) + 4 * gq + (t & 3)) * kD + cc];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const size_t off = base + (size_t)crow(orow(m)) * rp + cc;
            vraw[m] = v[off];
            oraw[m] = dout[off];
        }
    }
    __syncthreads();
    // ---- Gam = cumulative sum of g down the chunk: four threads per channel,
    // 16 rows each, then the totals of the earlier quarters
    {
        const int ch = tid & (kD - 1), qq = tid >> 7;
        float a = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) a += A2[16 * qq + r][ch];
        s.red[qq * kD + ch] = a;
        __syncthreads();
        float pre = 0.f;
        for (int j = 0; j < qq; ++j) pre += s.red[j * kD + ch];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            pre += A2[16 * qq + r][ch];
            A2[16 * qq + r][ch] = pre;
        }
        if (qq == 3) s.gl[ch] = pre;
    }
    __syncthreads();

    // the lane's own kh, qh and Gam, kept in registers to the end
    float gmo[16], kho[16], qho[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int r = orow(m);
        gmo[m] = A2[r][cc];
        kho[m] = A0[r][cc];
        qho[m] = A1[r][cc];
    }
    // -Kt = -e^Gam kh and Kb = e^(GL - Gam) kh, in 16-byte pieces, as hi / lo
    // fragments over kh and qh (read first: the layouts differ)
    {
        float4 kt4[4], kb4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tid + kCT * j, r = e >> 5, c4 = 4 * (e & 31);
            const float4 kh = ld4(&A0[r][c4]), gm = ld4(&A2[r][c4]), gl = ld4(&s.gl[c4]);
            const float4 et = exp4(gm);
            const float4 eb = exp4(make_float4(gl.x - gm.x, gl.y - gm.y, gl.z - gm.z, gl.w - gm.w));
            kt4[j] = scale4(mul4(et, kh), -1.f);
            kb4[j] = mul4(eb, kh);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tid + kCT * j, r = e >> 5, c4 = 4 * (e & 31);
            const int f = 4 * (r >> 4) + (c4 >> 5);
            b16::put_frag_hl(fh(0), fl(0), f, r & 15, (c4 >> 2) & 3, (c4 >> 4) & 1, kt4[j]);
            b16::put_frag_hl(fh(1), fl(1), f, r & 15, (c4 >> 2) & 3, (c4 >> 4) & 1, kb4[j]);
        }
    }
    __syncthreads();

    // ---- R = V - Kt S and dU = scale M^T dO + Kb dS' -------------------------
    // R starts from V, and the products add -Kt S
    float Ro[16], dUo[16];
    {
        f32x4 aR[4], aU[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            aU[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                aR[u][e] = orow(4 * u + e) < L ? RW::wid(vraw[4 * u + e]) : 0.f;
        }
        // -Kt S and Kb dS' on bf16 hi / lo pairs: k32 block sb takes the strip
        // slots of 16-row blocks 2 sb and 2 sb + 1
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            bf16x8 bsh, bsl, bdh, bdl;
            split_b(f32x4{scol[8 * sb], scol[8 * sb + 1], scol[8 * sb + 2], scol[8 * sb + 3]},
                    f32x4{scol[8 * sb + 4], scol[8 * sb + 5], scol[8 * sb + 6], scol[8 * sb + 7]},
                    bsh, bsl);
            split_b(f32x4{dcol[8 * sb], dcol[8 * sb + 1], dcol[8 * sb + 2], dcol[8 * sb + 3]},
                    f32x4{dcol[8 * sb + 4], dcol[8 * sb + 5], dcol[8 * sb + 6], dcol[8 * sb + 7]},
                    bdh, bdl);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                aR[u] = mma3(aR[u], b16::frag_at(fh(0), 4 * u + sb, lane),
                             b16::frag_at(fl(0), 4 * u + sb, lane), bsh, bsl);
                aU[u] = mma3(aU[u], b16::frag_at(fh(1), 4 * u + sb, lane),
                             b16::frag_at(fl(1), 4 * u + sb, lane), bdh, bdl);
            }
        }
        // M^T: A(i, kk) = N[kk][i], zero for kk < i, so row tile u takes blocks kb >= u
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            float o4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o4[e] = orow(4 * kb + e) < L ? scale * RW::wid(oraw[4 * kb + e]) : 0.f;
            const float4 bo = make_float4(o4[0], o4[1], o4[2], o4[3]);
            const int kr = 16 * kb + 4 * gq;
#pragma unroll
            for (int u = 0; u <= kb; ++u)
                mfma4(aU[u], make_float4(s.n[kr][16 * u + n], s.n[kr + 1][16 * u + n],
                                         s.n[kr + 2][16 * u + n], s.n[kr + 3][16 * u + n]),
                      bo);
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            Ro[m] = aR[m >> 2][m & 3];
            dUo[m] = aU[m >> 2][m & 3];
        }
    }
    __syncthreads();  // every read of Kt and Kb is done
    // S and dS' as row strips (S[cc][*], dS'[cc][*]): the column strips pass
    // through LDS, one matrix at a time, over the first two [64][132] arrays
    float4 srow[8], drow[8];
    {
        float(*const SS)[kPB] = s.big[0];  // [128][132]
#pragma unroll
        for (int t = 0; t < 32; ++t) SS[16 * (t >> 2) + 4 * gq + (t & 3)][cc] = scol[t];
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) srow[kb] = ld4(&SS[cc][16 * kb + 4 * gq]);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 32; ++t) SS[16 * (t >> 2) + 4 * gq + (t & 3)][cc] = dcol[t];
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) drow[kb] = ld4(&SS[cc][16 * kb + 4 * gq]);
        __syncthreads();
    }

    // ---- U = T R and dV = dR = T^T dU, T = X diag(beta), from registers ------
    float dRo[16];
    {
        f32x4 aX[4], aD[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) aX[u] = aD[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const float4 br = make_float4(Ro[4 * kb], Ro[4 * kb + 1], Ro[4 * kb + 2], Ro[4 * kb + 3]);
            const float4 bd =
                make_float4(dUo[4 * kb], dUo[4 * kb + 1], dUo[4 * kb + 2], dUo[4 * kb + 3]);
            const int kr = 16 * kb + 4 * gq;
            const float4 bb = ld4(&s.beta[kr]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                // X is lower triangular: U's row tile u takes blocks kb <= u, dR's kb >= u
                if (u >= kb) mfma4(aX[u], mul4(ld4(&s.x[16 * u + n][kr]), bb), br);
                if (u <= kb)
                    mfma4(aD[u], make_float4(s.x[kr][16 * u + n], s.x[kr + 1][16 * u + n],
                                             s.x[kr + 2][16 * u + n], s.x[kr + 3][16 * u + n]),
                          bd);
            }
        }
        float Uo[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int r = orow(m);
            dRo[m] = s.beta[r] * aD[m >> 2][m & 3];
            if (r < L) io_st(dv + base + (size_t)r * rp + cc, dRo[m]);
            Uo[m] = aX[m >> 2][m & 3];
        }
        stage_own(fh(0), fl(0), Ro, wv, n, gq);
        stage_own(fh(1), fl(1), dUo, wv, n, gq);
        stage_own(fh(2), fl(2), Uo, wv, n, gq);
    }
    __syncthreads();  // R, dU and U are in LDS

    // ---- the 64 x 64 products: wave w computes tiles (rt0, ct) and (rt0 + 2, ct)
    const int ct = wv & 3, rt0 = wv >> 2;
    // dT = lower-incl(dU R^T); dbeta_j = sum_i X_ij dT_ij; dX = dT diag(beta)
    float dXo[8];
    {
        f32x4 aT[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            const bf16x8 rh = b16::frag_at(fh(0), 4 * ct + sb, lane);
            const bf16x8 rl = b16::frag_at(fl(0), 4 * ct + sb, lane);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rt = rt0 + 2 * t;
                if (rt >= ct)
                    aT[t] = mma3(aT[t], b16::frag_at(fh(1), 4 * rt + sb, lane),
                                 b16::frag_at(fl(1), 4 * rt + sb, lane), rh, rl);
            }
        }
        const int j = 16 * ct + n;
        float pb = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * (rt0 + 2 * t) + 4 * gq + e;
                const float d = j <= i ? aT[t][e] : 0.f;
                pb = fmaf(s.x[i][j], d, pb);
                dXo[4 * t + e] = d * s.beta[j];
            }
        pb += __shfl_xor(pb, 16);
        pb += __shfl_xor(pb, 32);
        if (gq == 0) s.red[rt0 * kChunk + j] = pb;
    }
    __syncthreads();  // dT's reads of R and dU are done
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) DX[16 * (rt0 + 2 * t) + 4 * gq + e][16 * ct + n] = dXo[4 * t + e];
    {
        float so[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) so[m] = orow(m) < L ? scale * RW::wid(oraw[m]) : 0.f;
        stage_own(fh(1), fl(1), so, wv, n, gq);
    }
    if (tid < kChunk) s.dbeta[tid] = s.red[tid] + s.red[kChunk + tid];
    __syncthreads();  // dX and scale dO are in LDS
    // Y = X^T dX (Y_ij = sum_k X_ki dX_kj, k >= max(i, j)); dM = lower-incl(scale dO U^T)
    f32x4 aY[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    {
        f32x4 aM[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int kr = 16 * kb + 4 * gq;
            if (kb >= ct) {
                const float4 bX = make_float4(DX[kr][16 * ct + n], DX[kr + 1][16 * ct + n],
                                              DX[kr + 2][16 * ct + n], DX[kr + 3][16 * ct + n]);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int rt = rt0 + 2 * t;
                    if (kb >= rt)
                        mfma4(aY[t], make_float4(s.x[kr][16 * rt + n], s.x[kr + 1][16 * rt + n],
                                                 s.x[kr + 2][16 * rt + n], s.x[kr + 3][16 * rt + n]),
                              bX);
                }
            }
        }
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            const bf16x8 uh = b16::frag_at(fh(2), 4 * ct + sb, lane);
            const bf16x8 ul = b16::frag_at(fl(2), 4 * ct + sb, lane);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rt = rt0 + 2 * t;
                if (rt >= ct)
                    aM[t] = mma3(aM[t], b16::frag_at(fh(1), 4 * rt + sb, lane),
                                 b16::frag_at(fl(1), 4 * rt + sb, lane), uh, ul);
            }
        }
        // over N, whose last read was in dU
        const int j = 16 * ct + n;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * (rt0 + 2 * t) + 4 * gq + e;
                s.n[i][j] = j <= i ? aM[t][e] : 0.f;
            }
    }
    __syncthreads();  // Y's reads of dX are done
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) DX[16 * (rt0 + 2 * t) + 4 * gq + e][16 * ct + n] = aY[t][e];
    __syncthreads();  // Y is in LDS
    // dA = -strict-lower(Y X^T) (X_jk = 0 for k > j); dbeta_i += sum_j dA_ij P_ij;
    // dP = diag(beta) dA over P, each lane at its own elements
    {
        f32x4 aA[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (kb > ct) continue;
            const float4 bX = ld4(&s.x[16 * ct + n][16 * kb + 4 * gq]);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                if (rt0 + 2 * t >= ct) mfma4(aA[t], ld4(&DX[16 * (rt0 + 2 * t) + n][16 * kb + 4 * gq]), bX);
        }
        const int j = 16 * ct + n;
        float pr[8];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * (rt0 + 2 * t) + 4 * gq + e;
                const float a = j < i ? -aA[t][e] : 0.f;
                pr[4 * t + e] = a * s.p[i][j];
                s.p[i][j] = s.beta[i] * a;
            }
        row_sums(pr, n);  // lane n: value n / 2, i.e. tile n / 8, row 4 gq + (n / 2) % 4
        if ((n & 1) == 0) {
            const int vi = n >> 1;
            s.red[ct * kChunk + 16 * (rt0 + 2 * (vi >> 2)) + 4 * gq + (vi & 3)] = pr[0];
        }
    }
    __syncthreads();  // dA's reads of Y are done; dP, dM and the dbeta partials are in LDS
    stage_own(fh(0), fl(0), dRo, wv, n, gq);
    if (tid < kChunk) {
        float a = s.dbeta[tid];
        for (int j = 0; j < 4; ++j) a += s.red[j * kChunk + tid];
        s.dbeta[tid] = a;
    }
    __syncthreads();  // dR is in LDS

    // ---- dQt = scale dO S^T, dKt = -dR S^T, dKb = U dS'^T ----------------------
    // dqh = e^Gam dQt, dkh = e^Gam dKt + e^(GL - Gam) dKb,
    // dGam = Qt dQt + Kt dKt - Kb dKb; the last row of dGam also gets
    // sum_r Kb dKb (per channel, pl)
    float dqh[16], dkh[16], dgm[16], pl = 0.f;
    // dgamma = rowsum(dS' . S) at the lane's channel: over its row strips, then
    // over the four lanes of the channel; the last row of dGam gets gamma dgamma
    float dlast;
    {
        float a = 0.f;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
            a += srow[kb].x * drow[kb].x + srow[kb].y * drow[kb].y + srow[kb].z * drow[kb].z +
                 srow[kb].w * drow[kb].w;
        a += __shfl_xor(a, 16);
        a += __shfl_xor(a, 32);
        dlast = a * ex(s.gl[cc]);
    }
    {
        f32x4 aQ[4], aK[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) aQ[u] = aK[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            bf16x8 bh, bl;
            split_b(f32x4{srow[2 * sb].x, srow[2 * sb].y, srow[2 * sb].z, srow[2 * sb].w},
                    f32x4{srow[2 * sb + 1].x, srow[2 * sb + 1].y, srow[2 * sb + 1].z,
                          srow[2 * sb + 1].w},
                    bh, bl);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                aQ[u] = mma3(aQ[u], b16::frag_at(fh(1), 4 * u + sb, lane),
                             b16::frag_at(fl(1), 4 * u + sb, lane), bh, bl);
                aK[u] = mma3(aK[u], b16::frag_at(fh(0), 4 * u + sb, lane),
                             b16::frag_at(fl(0), 4 * u + sb, lane), bh, bl);
            }
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const float e = ex(gmo[m]), a = aQ[m >> 2][m & 3], bb = -aK[m >> 2][m & 3];
            dqh[m] = e * a;
            dkh[m] = e * bb;
            dgm[m] = e * fmaf(qho[m], a, kho[m] * bb);
        }
    }
    {
        f32x4 aB[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) aB[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            bf16x8 bh, bl;
            split_b(f32x4{drow[2 * sb].x, drow[2 * sb].y, drow[2 * sb].z, drow[2 * sb].w},
                    f32x4{drow[2 * sb + 1].x, drow[2 * sb + 1].y, drow[2 * sb + 1].z,
                          drow[2 * sb + 1].w},
                    bh, bl);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                aB[u] = mma3(aB[u], b16::frag_at(fh(2), 4 * u + sb, lane),
                             b16::frag_at(fl(2), 4 * u + sb, lane), bh, bl);
        }
        const float glc = s.gl[cc];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const float e = ex(glc - gmo[m]), a = aB[m >> 2][m & 3];
            const float t = e * kho[m] * a;
            dkh[m] = fmaf(e, a, dkh[m]);
            dgm[m] -= t;
            pl += t;
        }
        pl += __shfl_xor(pl, 16);
        pl += __shfl_xor(pl, 32);
    }

    // ---- the pairwise-decay terms of P and N ---------------------------------
    // row side:  a_rc = sum_i dP_ri E_ric kh_ic,  b_rc = sum_i dN_ri E_ric kh_ic
    // column side: c_ic = sum_r (dP_ri kh_rc + dN_ri qh_rc) E_ric
    // with E_ric = exp(Gam_rc - Gam_ic) (i <= r); then dkh += a + c, dqh += b,
    // dGam += kh a + qh b - kh c.  E is split about a reference row per
    // 16-row block, as in the forward: with g >= -5 each factor stays within
    // exp(+-75), finite in fp32.
    //   row side, i in block bk, reference e = 16 bk + 15:
    //     E = exp(Gam_r - Gam_e) exp(Gam_e - Gam_i), rows r >= 16 bk;
    //   column side, r in block bk, reference s0 = 16 bk:
    //     E = exp(Gam_r - Gam_s0) exp(Gam_s0 - Gam_i), rows i <= 16 bk + 15.
    // Each block's sums are a 16-deep product on the matrix cores whose B
    // operand (the block's factor rows, at the lane's channel) the lane forms
    // from its own slots 4 bk .. 4 bk + 3; the reference Gam comes from the
    // lane of the same channel that owns the reference row.
#pragma unroll
    for (int bk = 0; bk < 4; ++bk) {
        const float ge = __shfl(gmo[4 * bk + 3], n + 48);  // Gam at row 16 bk + 15
        const float gs = __shfl(gmo[4 * bk], n);           // Gam at row 16 bk
        float fr[4], fk[4], fq[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 4 * bk + e;
            fr[e] = kho[m] * ex(ge - gmo[m]);
            const float f = ex(gmo[m] - gs);
            fk[e] = kho[m] * f;
            fq[e] = qho[m] * f;
        }
        const float4 bR = make_float4(fr[0], fr[1], fr[2], fr[3]);
        const float4 bK = make_float4(fk[0], fk[1], fk[2], fk[3]);
        const float4 bQ = make_float4(fq[0], fq[1], fq[2], fq[3]);
        const int kr = 16 * bk + 4 * gq;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (u >= bk) {  // row side, rows of tile u >= the block
                f32x4 acn = {0.f, 0.f, 0.f, 0.f};
                mfma4(acc, ld4(&s.p[16 * u + n][kr]), bR);
                mfma4(acn, ld4(&s.n[16 * u + n][kr]), bR);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = 4 * u + e;
                    const float f = ex(gmo[m] - ge);
                    const float ta = f * acc[e], tb = f * acn[e];
                    dkh[m] += ta;
                    dqh[m] += tb;
                    dgm[m] = fmaf(kho[m], ta, fmaf(qho[m], tb, dgm[m]));
                }
            }
            if (u <= bk) {  // column side, rows of tile u <= the block
                f32x4 acx = {0.f, 0.f, 0.f, 0.f};
                const int i = 16 * u + n;
                mfma4(acx, make_float4(s.p[kr][i], s.p[kr + 1][i], s.p[kr + 2][i], s.p[kr + 3][i]), bK);
                mfma4(acx, make_float4(s.n[kr][i], s.n[kr + 1][i], s.n[kr + 2][i], s.n[kr + 3][i]), bQ);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = 4 * u + e;
                    const float tc = ex(gs - gmo[m]) * acx[e];
                    dkh[m] += tc;
                    dgm[m] = fmaf(-kho[m], tc, dgm[m]);
                }
            }
        }
    }

    // ---- the norms' backward, dg, and the stores ------------------------------
    // row dots qh . dqh and kh . dkh: over the 16 channels of the lane's column
    // tile, then over the 8 tiles in order
    {
        float aq[16], ak[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            aq[m] = qho[m] * dqh[m];
            ak[m] = kho[m] * dkh[m];
        }
        row_sums(aq, n);  // lane n: slot n
        row_sums(ak, n);
        const int r = orow(n);
        s.red[wv * kChunk + r] = aq[0];
        s.red[4 * kD + wv * kChunk + r] = ak[0];
    }
    __syncthreads();
    if (tid < kChunk) {
        float aq = 0.f, ak = 0.f;
        for (int w = 0; w < kCT / 64; ++w) {
            aq += s.red[w * kChunk + tid];
            ak += s.red[4 * kD + w * kChunk + tid];
        }
        s.dotq[tid] = aq;
        s.dotk[tid] = ak;
    } else if (tid < 2 * kChunk) {
        const int r = tid - kChunk;
        if (r < L) dbeta[((size_t)b * T + (size_t)cg * kChunk + r) * H + h] = s.dbeta[r];
    }
    // dg = reverse cumulative sum of dGam down the chunk; the last row also gets
    // gamma dgamma and sum_r Kb dKb.  Within the lane over e, then over the
    // lanes of the channel (gq) and the row tiles (u).
    {
        float sfx[16], gt[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float a = 0.f;
#pragma unroll
            for (int e = 3; e >= 0; --e) {
                a += dgm[4 * u + e];
                sfx[4 * u + e] = a;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) gt[u][j] = __shfl(a, n + 16 * j);
        }
        float after = dlast + pl;
#pragma unroll
        for (int u = 3; u >= 0; --u) {
            float later = 0.f, tot = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                later += j > gq ? gt[u][j] : 0.f;
                tot += gt[u][j];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 4 * u + e, r = orow(m);
                if (r < L) dg[base + (size_t)r * rp + cc] = sfx[m] + later + after;
            }
            after += tot;
        }
    }
    __syncthreads();  // the row dots are in LDS
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int r = orow(m);
        if (r >= L) continue;
        // qh = q / sqrt(|q|^2 + eps): dq = rq (dqh - qh (qh . dqh))
        io_st(dq + base + (size_t)r * rp + cc, s.rq[r] * fmaf(-qho[m], s.dotq[r], dqh[m]));
        io_st(dk + base + (size_t)r * rp + cc, s.rk[r] * fmaf(-kho[m], s.dotk[r], dkh[m]));
    }
}
}  // namespace

size_t chunk_bwd_segment_bytes_per_chunk(int B, int H) {
    return (size_t)B * H *
           (RF::BYTES + (2 * kStateFloats + (size_t)3 * kChunk * kChunk) * sizeof(float));
}

namespace {
// Workspace of a segment of nch chunks: records, then the states entering the
// chunks, the state gradients leaving them, and X, P and N of each chunk.
struct SegWs {
    uint8_t* rec;
    float *states, *dsn, *xs;
    SegWs(void* ws, int B, int H, int nch) {
        const size_t n = (size_t)B * H * nch;
        rec = static_cast<uint8_t*>(ws);
        states = reinterpret_cast<float*>(rec + n * RF::BYTES);
        dsn = states + n * kStateFloats;
        xs = dsn + n * kStateFloats;
    }
};
}  // namespace

template <typename IO>
hipError_t launch_chunk_fwd_state(const IO* q, const IO* k, const IO* v, const float* g,
                                  const float* beta, const float* h_in, float* h_out, int B,
                                  int T, int H, int chunk0, int nch, void* ws,
                                  const WaitCtl& wait, hipStream_t stream) {
    const SegWs w(ws, B, H, nch);
    hipError_t e = launch_chunk_prep_f32(q, k, g, beta, B, T, H, chunk0, nch, w.rec, stream);
    if (e != hipSuccess) return e;
    const unsigned nscan = (unsigned)((int64_t)B * H * kScanSlices);
    hipLaunchKernelGGL(kda_bwd_state_scan_kernel<IO>, dim3(nscan), dim3(kScanThreads), 0, stream,
                       w.rec, v, h_in, w.states, h_out, T, H, chunk0, nch, wait);
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_chunk_bwd_segment(const IO* q, const IO* k, const IO* v, const float* g,
                                    const float* beta, float scale, const float* h_in,
                                    const IO* dout, const float* dS_in, IO* dq, IO* dk, IO* dv,
                                    float* dg, float* dbeta, float* dS_out, int B, int T, int H,
                                    int chunk0, int nch, void* ws, const WaitCtl& wait,
                                    hipStream_t stream) {
    const SegWs w(ws, B, H, nch);
    hipError_t e =
        launch_chunk_prep_f32(q, k, g, beta, B, T, H, chunk0, nch, w.rec, stream, w.xs);
    if (e != hipSuccess) return e;
    const unsigned nscan = (unsigned)((int64_t)B * H * kScanSlices);
    hipLaunchKernelGGL(kda_bwd_state_scan_kernel<IO>, dim3(nscan), dim3(kScanThreads), 0, stream,
                       w.rec, v, h_in, w.states, nullptr, T, H, chunk0, nch, wait);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(kda_bwd_grad_scan_kernel<IO>, dim3(nscan), dim3(kScanThreads), 0, stream,
                       w.rec, dout, dS_in, w.dsn, dS_out, scale, T, H, chunk0, nch, wait);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t n = (size_t)B * H * nch;
    hipLaunchKernelGGL(kda_bwd_chunk_kernel<IO>, dim3((unsigned)n), dim3(kCT), 0, stream, q, k, v,
                       g, beta, dout, w.states, w.dsn, w.xs, scale, T, H, chunk0, nch, dq,
                       dk, dv, dg, dbeta);
    return hipGetLastError();
}

#define KDA_INST_BWD(IO)                                                                        \
    template hipError_t launch_chunk_fwd_state<IO>(const IO*, const IO*, const IO*,              \
                                                   const float*, const float*, const float*,     \
                                                   float*, int, int, int, int, int, void*,       \
                                                   const WaitCtl&, hipStream_t);                 \
    template hipError_t launch_chunk_bwd_segment<IO>(                                            \
        const IO*, const IO*, const IO*, const float*, const float*, float, const float*,        \
        const IO*, const float*, IO*, IO*, IO*, float*, float*, float*, int, int, int, int, int, \
        void*, const WaitCtl&, hipStream_t);
KDA_INST_BWD(float)
KDA_INST_BWD(uint16_t)
#undef KDA_INST_BWD

}  // namespace kda
