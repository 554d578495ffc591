// Chunkwise KDA prefill for bf16 q/k/v/o in two kernels (the pages' chunk_kda).
//
// The recurrence (Kimi-K3 深度解析 blog, section 三: decay the state per key
// channel, predict v from the decayed state, write beta times the error along
// the key; read out with the L2-normalised query, 深入 Kimi-K3 thread, KDA
// paragraph) is evaluated 64 tokens at a time.  For one chunk of tokens
// r = 0..63 entering with state S (key channel x value channel), with
// Gam_r = sum_{s<=r} g_s per channel:
//   Kt_r = exp(Gam_r) kh_r,  Qt_r = exp(Gam_r) qh_r,
//   Kb_r = exp(Gam_63 - Gam_r) kh_r,  gamma = exp(Gam_63),
//   A = strict-lower(diag(beta) (KK)),  M = lower-incl(QK), where
//   (KK)_ri = sum_c kh_rc kh_ic exp(Gam_rc - Gam_ic) and (QK) likewise,
//   T = (I + A)^-1 diag(beta).
// Token by token the errors u_r = beta_r (v_r - prediction_r) stack into
//   U = T (V - Kt S),   O = scale (Qt S + M U),   S <- Diag(gamma) S + Kb^T U,
// an exact rearrangement of the recurrence.  The -5 lower bound on the
// log-decay (ai-pulse-lab summary of the technical report, KDA paragraph)
// keeps every factor of the 16x16 diagonal blocks of KK and QK finite, so all
// of them are dense matrix-core products: exp(Gam_r - Gam_i) is formed as a
// row factor times a column factor about the last token of each 16-token
// column block (row factors up to exp(75), column factors <= 1).
//
// prep (kda_prep16_kernel): one workgroup per (batch, head, chunk), all chunks
//   in parallel.  It normalises q and k, forms the decay sums and factor
//   tables, the KK / QK blocks on MFMA, the inverse of I + A in fp32, and
//   writes the chunk's record: Kt, Qt, Kb^T, M (bf16), T (bf16 hi + lo) and
//   gamma, laid out as the scan kernel's LDS image.
// scan (kda_scan16_kernel): one workgroup per (batch, head, 64 value columns),
//   walking the chunks in order.  Four loader waves copy each record from
//   global memory into LDS one chunk ahead; four scan waves each keep a
//   128 x 16 fp32 slice of the state in registers and run the chunk's products
//   on MFMA.  The two roles hand the record over through LDS counters (Kt / Qt
//   / V first, the rest second, the rest in two buffers by chunk parity), so
//   the scan waves never wait for a workgroup barrier.
//
// Precision: Kt, Qt, Kb, M and the state enter the products as bf16; V - Kt S,
// T and U as bf16 hi + lo pairs (about 16 mantissa bits, three products per
// pair, two where the other factor is plain bf16); accumulation is fp32.  M
// feeds only the output, so its rounding does not build up in the state.
#include "kda_bf16.hpp"
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {
namespace {
using namespace b16;

constexpr int kSlices = 2;             // value-column slices per head
constexpr int kCols = kD / kSlices;    // value columns per scan workgroup
// Row pitch of the V slice in the scan's LDS: 34 dwords.  A pitch of 2 mod 4
// dwords makes the 8-byte fragment reads of 16 rows x 4 k-groups
// conflict-free on gfx950 (measured: about 110-120 B/clk per CU, against 62
// at 32 or 36 dwords).
constexpr int VP = kCols + 4;
constexpr int SP = kChunk + 1;         // fp32 pitch of A and X in the prep kernel

// decay tables per channel (exp of sums of the four block totals tau_a):
//   EP_a = exp(sum_{a'<a} tau), EK_a = exp(sum_{a'>a} tau), IE_a = exp(-tau_a),
//   TF(a,b) = exp(sum_{b<a'<a} tau) for a - b >= 2, and gamma.
enum { kEP = 0, kEK = 4, kIE = 8, kTF20 = 12, kTF30 = 13, kTF31 = 14, kGam = 15, kTabs = 16 };

// Record of one (batch, head, chunk) in global memory: the image of the scan
// kernel's LDS, so that the scan's loaders copy it verbatim.  Every matrix is
// stored as the k32 operand fragments the scan's products read: a fragment is
// 16 rows x 32 k of bf16, 1 KB, lane (n, g) of the reading wave at byte
// 16 (n + 16 g) holding row n with k = k0 + 4g + e (values 0..3) and
// k0 + 16 + 4g + e (values 4..7), so that every fragment read is one
// conflict-free 16-byte LDS read per lane.
//   Kt, Qt:  fragment 4 rt + s = tokens 16 rt .., channels 32 s ..   (16 KB each)
//   Kb^T:    fragment 2 t + s2 = channels 16 t .., tokens 32 s2 ..  (16 KB)
//   T hi, T lo, M (5 KB each): the six fragments (rt, s2) = (0,0)
//     (1,0) (2,0) (2,1) (3,0) (3,1) of the lower-triangular [token][token]
//     matrix; (0,0) and (2,1) have zero values 4..7 (blocks above the
//     diagonal) and are stored as half fragments, 8 bytes per lane;
//   gamma [128] fp32.
struct Rec16 {
    static constexpr size_t kFrag = 1024;
    static constexpr size_t KT = 0;
    static constexpr size_t QT = KT + 16 * kFrag;
    static constexpr size_t KB = QT + 16 * kFrag;
    static constexpr size_t TM = KB + 16 * kFrag;
    static constexpr size_t kTM = 5 * kFrag;                 // one of the three matrices
    static constexpr size_t G = TM + 3 * kTM;
    static constexpr size_t BYTES = G + kD * 4;
};
static_assert(Rec16::BYTES % 256 == 0, "records stay 256-byte aligned");
// the scan's loaders move a record as 16-byte pieces: 2048 of Kt / Qt, then
// the rest, 1024 of Kb^T, 960 of T / M and 32 of gamma: 7 per thread and 224
// more, 256 threads
constexpr int kRestFull = 7, kRestTail = 224;
static_assert(Rec16::KB / 16 == 2048 && Rec16::G / 16 + 32 == Rec16::BYTES / 16 &&
                  (Rec16::BYTES - Rec16::KB) / 16 == kRestFull * 256 + kRestTail,
              "loader piece counts match the record layout");

// fragment f = 0..5 of a T / M matrix: (rt, s2) and byte offset in the matrix
__host__ __device__ constexpr int tm_rt(int f) { return f < 2 ? f : 2 + ((f - 2) >> 1); }
__host__ __device__ constexpr int tm_s2(int f) { return f < 2 ? 0 : (f - 2) & 1; }
__host__ __device__ constexpr bool tm_half(int f) { return f == 0 || f == 3; }
__host__ __device__ constexpr int tm_off(int f) {
    return f == 0 ? 0 : f == 1 ? 512 : f == 2 ? 1536 : f == 3 ? 2560 : f == 4 ? 3072 : 4096;
}
static_assert(tm_off(5) + 1024 == (int)Rec16::kTM, "T / M fragment offsets");

// Short convolution + SiLU of the 8 channels cb.. of token tok = t0 + n of a
// [B, T, H, 128] bf16 tensor x, where the 16 lanes n = 0..15 of each DPP row
// hold 16 consecutive tokens with the same channels: silu(sum_j w_j
// x_{tok-3+j}) per channel, taps wr [8][4] of these channels (tap 3 = the
// current token),
// tokens before the sequence from st ([B][3][H][128] bf16, the raw tokens
// -3 .. -1) or zero.  Each lane loads its own row; lanes 13..15 also load the
// row 16 tokens back.  A row rotation by j then hands lane n the row of lane
// n - j, or, for n < j, the back row of lane n - j + 16, i.e. token tok - j
// in both cases.  Every lane of the row must call this; rows past the end
// return zeros.  Returns the 8 results as bf16.
__device__ __forceinline__ u32x4 conv_silu8_row16(const uint16_t* x, const float* wr,
                                                  const uint16_t* st, int b, int64_t tok, int n,
                                                  int T, int H, int h, int cb) {
    const int64_t tc = tok < T ? tok : T - 1;
    const u32x4 xr =
        *reinterpret_cast<const u32x4*>(x + (((int64_t)b * T + tc) * H + h) * kD + cb);
    u32x4 hr = {0u, 0u, 0u, 0u};
    const int64_t th = tok - 16;  // >= -3: only the first block of a sequence reaches back
    if (n >= 13 && th < T) {      // a back row at or past the end feeds only rows past it
        if (th >= 0)
            hr = *reinterpret_cast<const u32x4*>(x + (((int64_t)b * T + th) * H + h) * kD + cb);
        else if (st)
            hr = *reinterpret_cast<const u32x4*>(st + (((int64_t)b * 3 + (3 + th)) * H + h) * kD +
                                                 cb);
    }
    // the 3 earlier tokens of each register (all lanes take part in the
    // rotations); then, on rows before the end only, the filter (the branch
    // also keeps the register demand of the caller within its budget)
    uint32_t xa[4][4];  // xa[r][j]: register r of token tok - 3 + j
#pragma unroll
    for (int r2 = 0; r2 < 4; ++r2) {
        xa[r2][3] = xr[r2];
#define KDA_ROW_ROR(d)                                                                      \
        xa[r2][3 - (d)] = (uint32_t)__builtin_amdgcn_update_dpp(                            \
            0, (int)(n >= 16 - (d) ? hr[r2] : xr[r2]), 0x120 + (d), 0xf, 0xf, false)  /* row_ror:d */
        KDA_ROW_ROR(1);
        KDA_ROW_ROR(2);
        KDA_ROW_ROR(3);
#undef KDA_ROW_ROR
    }
    u32x4 res = {0u, 0u, 0u, 0u};
    if (tok >= T) return res;
#pragma unroll
    for (int r2 = 0; r2 < 4; ++r2) {
        const uint32_t* xj = xa[r2];
        float y[2];
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
            const f32x4 we = *reinterpret_cast<const f32x4*>(wr + 4 * (2 * r2 + hi));
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float xv =
                    __builtin_bit_cast(float, hi ? (xj[j] & 0xffff0000u) : (xj[j] << 16));
                acc += we[j] * xv;
            }
            y[hi] = acc * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * acc));
        }
        res[r2] = pack2(y[0], y[1]);
    }
    return res;
}

}  // namespace

size_t chunk16_record_bytes() { return Rec16::BYTES; }
int chunk16_slices() { return kSlices; }

// ---------------------------------------------------------------------------
// prep: wave p owns chunk rows 16p..16p+15; lane (n, gq) owns row r = 16p + n
// and the 32 channels 32s + 8gq + e (s = 0..3, e = 0..7), i.e. its A-operand
// fragments of the four k32 steps over the 128 channels.  G16: g arrives as
// bf16 (widened to fp32 on load) instead of fp32.  CONV: q and k are the raw
// values before the short convolution, which is applied on load (the
// filtered values rounded to bf16).
// ---------------------------------------------------------------------------
template <bool G16, bool CONV>
__global__ __launch_bounds__(256, 3) void kda_prep16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const void* __restrict__ g,
    const float* __restrict__ beta, int T, int H, int chunk0, int nchunks,
    uint8_t* __restrict__ ws, ConvArgs conv) {
    __shared__ __align__(16) float tau_s[4][kD];      // block totals of g (log2 units)
    __shared__ __align__(16) float tab_s[kTabs][kD];  // factor tables
    __shared__ float beta_s[kChunk];
    // The column operands of KK / QK and X = (I + A)^-1 share one area (a
    // barrier separates their uses), so that three workgroups fit on a CU
    // (43 KB of LDS each).
    __shared__ __align__(16) float u1_s[kChunk * SP];
    __shared__ float a_s[kChunk * SP];                 // diag(beta) strict-lower KK
    // CONV: the short convolution's taps of q and k for this head, [2][128][4]
    __shared__ __align__(16) float taps_s[CONV ? 2 * kD * 4 : 4];
    static_assert(sizeof(bf16x8) * 4 * 4 * 64 <= sizeof(float) * kChunk * SP,
                  "column operands fit the shared area");
    bf16x8 (*zf_s)[4][64] = reinterpret_cast<bf16x8 (*)[4][64]>(u1_s);
    float* x_s = u1_s;
    // Kb^T passes through a_s before a_s holds A: fragment f (1 KB) lies in
    // the rows of wave f / 4 (16 rows of SP floats, 4,160 bytes each wave)
    uint8_t* kb_stage = reinterpret_cast<uint8_t*>(a_s);
    auto kb_stage_off = [](int f) { return 16 * SP * 4 * (f >> 2) + 1024 * (f & 3); };
    static_assert(16 * SP * 4 >= 4 * 1024, "a wave's Kb^T fragments fit its rows of a_s");

    // Chunk-major order, XCD-aware: workgroups are dealt round-robin to the 8
    // XCDs, so the k-th workgroup of XCD x takes chunk k / (BH / 8) and head
    // x BH / 8 + k % (BH / 8).  The heads of one chunk then run together, and
    // consecutive heads on one XCD: their q / k / g rows are one contiguous
    // stream and a cache line of beta (32 heads of one token) is fetched by
    // few XCDs instead of once per head.  Records are stored chunk-major too.
    const int BH = gridDim.x / nchunks;
    int cl, bh;
    if (BH % 8 == 0) {
        const int id = blockIdx.x, hx = BH / 8, k = id / 8;
        cl = k / hx;
        bh = (id % 8) * hx + k % hx;
    } else {
        cl = blockIdx.x / BH;
        bh = blockIdx.x % BH;
    }
    const int h = bh % H, b = bh / H;
    const int c = chunk0 + cl;
    uint8_t* rec = ws + ((size_t)cl * BH + bh) * Rec16::BYTES;

    const int tid = threadIdx.x, lane = tid & 63;
    const int p = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, gq = lane >> 4;
    const int r = 16 * p + n;
    const int64_t tok = (int64_t)c * kChunk + r;
    const bool valid = tok < T;
    const int64_t rowoff = (((int64_t)b * T + (valid ? tok : 0)) * H + h) * kD;

    // ---- load the lane's row: 32 channels of q, k (bf16 pairs) and g ---------
    u32x4 pq[4], pk[4];
    f32x4 pg[8];
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    const f32x4 zf4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int cb = 32 * s + 8 * gq;
        if constexpr (!CONV) {
            pq[s] = valid ? *reinterpret_cast<const u32x4*>(q + rowoff + cb) : z4;
            pk[s] = valid ? *reinterpret_cast<const u32x4*>(k + rowoff + cb) : z4;
        }
        if constexpr (G16) {
            const u32x4 x = valid
                ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(g) + rowoff + cb)
                : z4;
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                pg[2 * s + w] = f32x4{__builtin_bit_cast(float, x[2 * w] << 16),
                                      __builtin_bit_cast(float, x[2 * w] & 0xffff0000u),
                                      __builtin_bit_cast(float, x[2 * w + 1] << 16),
                                      __builtin_bit_cast(float, x[2 * w + 1] & 0xffff0000u)};
            }
        } else {
            const float* gf = static_cast<const float*>(g);
            pg[2 * s] = valid ? *reinterpret_cast<const f32x4*>(gf + rowoff + cb) : zf4;
            pg[2 * s + 1] = valid ? *reinterpret_cast<const f32x4*>(gf + rowoff + cb + 4) : zf4;
        }
    }
    const float bet = valid ? beta[((int64_t)b * T + tok) * H + h] : 0.f;
    if constexpr (CONV) {
        // the taps into LDS (one 16-byte piece per thread) while the g loads
        // are in flight, then q and k through the filter
        {
            const float* wsrc = (tid < kD ? conv.wq : conv.wk) + ((size_t)h * kD + (tid & (kD - 1))) * 4;
            *reinterpret_cast<f32x4*>(&taps_s[4 * tid]) = *reinterpret_cast<const f32x4*>(wsrc);
        }
        __syncthreads();
        const size_t st_n = (size_t)conv.B * 3 * H * kD;  // one tensor's state
        const uint16_t* sq = conv.state;
        const uint16_t* sk = conv.state ? conv.state + st_n : nullptr;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int cb = 32 * s + 8 * gq;
            pq[s] = conv_silu8_row16(q, &taps_s[4 * cb], sq, b, tok, n, T, H, h, cb);
            pk[s] = conv_silu8_row16(k, &taps_s[4 * (kD + cb)], sk, b, tok, n, T, H, h, cb);
        }
    }

    // ---- norms of q and k; in-block cumsum of g over the 16 rows -------------
    float ssq = 0.f, ssk = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float q0 = __builtin_bit_cast(float, pq[s][w] << 16);
            const float q1 = __builtin_bit_cast(float, pq[s][w] & 0xffff0000u);
            const float k0 = __builtin_bit_cast(float, pk[s][w] << 16);
            const float k1 = __builtin_bit_cast(float, pk[s][w] & 0xffff0000u);
            ssq += q0 * q0 + q1 * q1;
            ssk += k0 * k0 + k1 * k1;
        }
    }
    ssq += __shfl_xor(ssq, 16);
    ssk += __shfl_xor(ssk, 16);
    ssq += __shfl_xor(ssq, 32);
    ssk += __shfl_xor(ssk, 32);
    const float iq = __builtin_amdgcn_rsqf(ssq + kNormEps);
    const float ik = __builtin_amdgcn_rsqf(ssk + kNormEps);
    float lam[32];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            lam[8 * s + e] = row16_inclusive_scan(pg[2 * s][e] * kLog2e);
            lam[8 * s + 4 + e] = row16_inclusive_scan(pg[2 * s + 1][e] * kLog2e);
        }
    }
    if (n == 15) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) tau_s[p][32 * s + 8 * gq + e] = lam[8 * s + e];
    }
    if (gq == 0) beta_s[r] = bet;
    __syncthreads();

    // ---- factor tables ---------------------------------------------------------
#pragma unroll
    for (int m = 0; m < kTabs / 2; ++m) {
        const int idx = tid + 256 * m, tb = idx >> 7, ch = idx & 127;
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
            default: x = t0 + t1 + t2 + t3; break;  // gamma
        }
        tab_s[tb][ch] = __builtin_amdgcn_exp2f(x);
    }
    __syncthreads();

    // ---- decay factors; Kt, Qt and Kb^T of the record ------------------------
    // e0 = exp(Gam_r - Gam_{16p-1}) <= 1, z = exp(Gam_{16p+15} - Gam_r) <= 1;
    // rk0 = kh e0 and rq0 = qh e0 are the KK / QK row operands before the
    // per-block factor; Kt = rk0 EP_p, Qt = rq0 EP_p, Kb = kh z EK_p.
    // Channels 8gq .. 8gq+3 and 8gq+4 .. +7 of k-step s land in lanes
    // 2 (gq & 1) and 2 (gq & 1) + 1 of fragment (p, s), in the upper half of
    // the values for gq >= 2.  Kb is transposed on the matrix cores: a product
    // with a 0/1 selection matrix as B (value e of lane (j, gq) is 1 where
    // 8 gq + e = 16 h + j) returns lane (j, g) the tokens 16p + 4g .. +3 of
    // channel 32s + 16h + j, exactly: 8 bytes of Kb^T fragment (2s + h, p / 2).
    // Lanes L and L + 32 (gq and gq + 2) hold the two 8-byte halves of the
    // same 16-byte fragment slots, for the slot at +0 (values of k0 + 4g ..)
    // and the one at +256 (k0 + 16 + 4g ..).  A swap of the upper 32 lanes of
    // one register with the lower 32 of another hands lanes gq < 2 both halves
    // of the +0 slot and lanes gq >= 2 both halves of the +256 slot, so that
    // each lane stores one 16-byte piece.
    auto store_pair = [](uint8_t* dst, const uint32_t (&w)[4]) {
        const auto a = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
        const auto c = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
        *reinterpret_cast<u32x4*>(dst) = u32x4{a[0], c[0], a[1], c[1]};
    };
    float rk0[32], rq0[32];
    {
        const size_t kq0 = (size_t)(16 * (2 * (gq & 1)) + n) * 16 + 256 * (gq >> 1);
        uint8_t* ktg = rec + Rec16::KT + 4 * p * Rec16::kFrag + kq0;
        uint8_t* qtg = rec + Rec16::QT + 4 * p * Rec16::kFrag + kq0;
        // Kb^T halves go to LDS first (kb_stage); the workgroup barrier below
        // completes every 16-byte slot
        uint8_t* kbl = kb_stage + (n + 16 * gq) * 16 + 8 * (p & 1);
        bf16x8 sel[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            u32x4 u;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                u[w] = (8 * gq + 2 * w == 16 * hh + n ? 0x3f80u : 0u) |
                       (8 * gq + 2 * w + 1 == 16 * hh + n ? 0x3f800000u : 0u);
            sel[hh] = __builtin_bit_cast(bf16x8, u);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int cb = 32 * s + 8 * gq;
            float ep[8], ek[8], ta[8], zc[8];
            *reinterpret_cast<f32x4*>(ep) = *reinterpret_cast<const f32x4*>(&tab_s[kEP + p][cb]);
            *reinterpret_cast<f32x4*>(ep + 4) = *reinterpret_cast<const f32x4*>(&tab_s[kEP + p][cb + 4]);
            *reinterpret_cast<f32x4*>(ek) = *reinterpret_cast<const f32x4*>(&tab_s[kEK + p][cb]);
            *reinterpret_cast<f32x4*>(ek + 4) = *reinterpret_cast<const f32x4*>(&tab_s[kEK + p][cb + 4]);
            *reinterpret_cast<f32x4*>(ta) = *reinterpret_cast<const f32x4*>(&tau_s[p][cb]);
            *reinterpret_cast<f32x4*>(ta + 4) = *reinterpret_cast<const f32x4*>(&tau_s[p][cb + 4]);
            uint32_t ktw[4], qtw[4], kbw[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float kh0 = __builtin_bit_cast(float, pk[s][w] << 16) * ik;
                const float kh1 = __builtin_bit_cast(float, pk[s][w] & 0xffff0000u) * ik;
                const float qh0 = __builtin_bit_cast(float, pq[s][w] << 16) * iq;
                const float qh1 = __builtin_bit_cast(float, pq[s][w] & 0xffff0000u) * iq;
                const int j = 8 * s + 2 * w;
                const float e00 = __builtin_amdgcn_exp2f(lam[j]);
                const float e01 = __builtin_amdgcn_exp2f(lam[j + 1]);
                const float z0 = __builtin_amdgcn_exp2f(ta[2 * w] - lam[j]);
                const float z1 = __builtin_amdgcn_exp2f(ta[2 * w + 1] - lam[j + 1]);
                zc[2 * w] = kh0 * z0;
                zc[2 * w + 1] = kh1 * z1;
                rk0[j] = kh0 * e00;
                rk0[j + 1] = kh1 * e01;
                rq0[j] = qh0 * e00;
                rq0[j + 1] = qh1 * e01;
                ktw[w] = pack2(rk0[j] * ep[2 * w], rk0[j + 1] * ep[2 * w + 1]);
                qtw[w] = pack2(rq0[j] * ep[2 * w], rq0[j + 1] * ep[2 * w + 1]);
                kbw[w] = pack2(zc[2 * w] * ek[2 * w], zc[2 * w + 1] * ek[2 * w + 1]);
            }
            store_pair(ktg + s * Rec16::kFrag, ktw);
            store_pair(qtg + s * Rec16::kFrag, qtw);
            zf_s[p][s][lane] = pack8(zc);
            const bf16x8 kbf = __builtin_bit_cast(bf16x8, u32x4{kbw[0], kbw[1], kbw[2], kbw[3]});
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const f32x4 t = mma(f32x4{0.f, 0.f, 0.f, 0.f}, kbf, sel[hh]);
                *reinterpret_cast<uint2*>(kbl + kb_stage_off(2 * (2 * s + hh) + (p >> 1))) =
                    uint2{pack2(t[0], t[1]), pack2(t[2], t[3])};
            }
        }
    }
    __syncthreads();
    // Kb^T fragments 4p .. 4p + 3 from the staging area (this wave's own rows
    // of a_s, which it writes only at the end of the next phase) to the
    // record, one 16-byte piece per lane each
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int fr = 4 * p + f;
        *reinterpret_cast<u32x4*>(rec + Rec16::KB + fr * Rec16::kFrag + lane * 16) =
            *reinterpret_cast<const u32x4*>(kb_stage + kb_stage_off(fr) + lane * 16);
    }

    // ---- KK and QK blocks of row block p against column blocks cb <= p ---------
    // row factor exp(Gam_r - Gam_{16cb+15}) = e0 * f with f = IE_p (cb = p),
    // 1 (cb = p - 1), TF(p, cb) otherwise.  The products are taken transposed
    // (column operand as A), so that a lane ends up with row r and the four
    // consecutive columns 16cb + 4g + e.
    f32x4 Mt[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        Mt[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (cb > p) continue;
        const int tix = (cb == p) ? kIE + p : (p - cb == 2) ? (p == 2 ? kTF20 : kTF31) : kTF30;
        const bool unit = (cb == p - 1);
        f32x4 accK = {0.f, 0.f, 0.f, 0.f}, accQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int cbase = 32 * s + 8 * gq;
            bf16x8 rk, rq;
            if (unit) {
                rk = pack8(rk0 + 8 * s);
                rq = pack8(rq0 + 8 * s);
            } else {
                float f[8], tk[8], tq[8];
                *reinterpret_cast<f32x4*>(f) = *reinterpret_cast<const f32x4*>(&tab_s[tix][cbase]);
                *reinterpret_cast<f32x4*>(f + 4) = *reinterpret_cast<const f32x4*>(&tab_s[tix][cbase + 4]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    tk[e] = rk0[8 * s + e] * f[e];
                    tq[e] = rq0[8 * s + e] * f[e];
                }
                rk = pack8(tk);
                rq = pack8(tq);
            }
            const bf16x8 fz = zf_s[cb][s][lane];
            accK = mma(accK, fz, rk);
            accQ = mma(accQ, fz, rq);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ci = 16 * cb + 4 * gq + e;
            const bool strict = (cb < p) || (ci < r);
            const bool incl = (cb < p) || (ci <= r);
            a_s[r * SP + ci] = strict ? bet * accK[e] : 0.f;
            Mt[cb][e] = incl ? accQ[e] : 0.f;
        }
    }
    __syncthreads();

    // ---- X = (I + A)^-1: diagonal blocks by forward substitution --------------
    {
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float s = 0.f;
#pragma unroll
            for (int cc = 0; cc < rr; ++cc) s += a_s[(16 * p + rr) * SP + 16 * p + cc] * x[cc];
            x[rr] = (rr == n) ? 1.f : -s;
        }
        if (gq == 0) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) x_s[(16 * p + rr) * SP + 16 * p + n] = x[rr];
        }
    }
    __syncthreads();
    // off-diagonal blocks by distance: X_ab = -X_aa sum_{c=b}^{a-1} A_ac X_cb
    // (fp32 matrix-core products, 16x16x4)
#pragma unroll
    for (int d = 1; d < 4; ++d) {
        if (p >= d) {
            const int a = p, bb = p - d;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int cc = bb; cc < a; ++cc) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        a_s[(16 * a + n) * SP + 16 * cc + 4 * gq + e],
                        x_s[(16 * cc + 4 * gq + e) * SP + 16 * bb + n], acc, 0, 0, 0);
            }
            f32x4 xab = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                xab = __builtin_amdgcn_mfma_f32_16x16x4f32(x_s[(16 * a + n) * SP + 16 * a + 4 * gq + e],
                                                          acc[e], xab, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) x_s[(16 * a + 4 * gq + e) * SP + 16 * bb + n] = -xab[e];
        }
        __syncthreads();
    }

    // ---- the rest of the record -------------------------------------------------
    // T = X diag(beta) (zero above the diagonal) as hi / lo and M: row r,
    // columns 16ct + 4g .. +3 per lane, lower blocks (p, ct <= p) only: value
    // half ct & 1 of lane (n, g) of fragment (p, ct / 2).  Column blocks 2cp
    // and 2cp + 1 fill the two halves of a lane's 16 bytes of a full
    // fragment, stored together; a half fragment (cp = p / 2 for even p) is
    // 8 bytes per lane.
    {
        uint8_t* tm = rec + Rec16::TM;
#pragma unroll
        for (int cp = 0; cp < 2; ++cp) {
            if (2 * cp > p) continue;
            const int f = p < 2 ? p : 2 + 2 * (p - 2) + cp;
            const bool half = tm_half(f);
            uint32_t th[4], tl[4], mh[4];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int ct = 2 * cp + hh;
                if (hh == 1 && half) continue;
                float tv[4], mv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int col = 16 * ct + 4 * gq + e;
                    tv[e] = (col <= r) ? x_s[r * SP + col] * beta_s[col] : 0.f;
                    mv[e] = Mt[ct][e];
                }
                uint2 h2, l2;
                split4(tv, h2, l2);
                th[2 * hh] = h2.x;
                th[2 * hh + 1] = h2.y;
                tl[2 * hh] = l2.x;
                tl[2 * hh + 1] = l2.y;
                mh[2 * hh] = pack2(mv[0], mv[1]);
                mh[2 * hh + 1] = pack2(mv[2], mv[3]);
            }
            if (half) {
                const size_t off = tm_off(f) + (size_t)lane * 8;
                *reinterpret_cast<uint2*>(tm + 0 * Rec16::kTM + off) = uint2{th[0], th[1]};
                *reinterpret_cast<uint2*>(tm + 1 * Rec16::kTM + off) = uint2{tl[0], tl[1]};
                *reinterpret_cast<uint2*>(tm + 2 * Rec16::kTM + off) = uint2{mh[0], mh[1]};
            } else {
                const size_t off = tm_off(f) + (size_t)lane * 16;
                *reinterpret_cast<u32x4*>(tm + 0 * Rec16::kTM + off) = u32x4{th[0], th[1], th[2], th[3]};
                *reinterpret_cast<u32x4*>(tm + 1 * Rec16::kTM + off) = u32x4{tl[0], tl[1], tl[2], tl[3]};
                *reinterpret_cast<u32x4*>(tm + 2 * Rec16::kTM + off) = u32x4{mh[0], mh[1], mh[2], mh[3]};
            }
        }
    }
    if (p == 0) {
        float* gg = reinterpret_cast<float*>(rec + Rec16::G);
        gg[lane] = tab_s[kGam][lane];
        gg[lane + 64] = tab_s[kGam][lane + 64];
    }
}

// ---------------------------------------------------------------------------
// scan: waves 0..3 load records, waves 4..7 scan (wave w owns value columns
// j0 .. j0+15 of the state as eight 16x16 accumulator tiles, key rows
// 16t + 4g + e, column j0 + n).  k order of every product: values 0..3 of a
// lane carry k = k0 + 4g + e, values 4..7 carry k0 + 16 + 4g + e, i.e. the
// rows of accumulator tiles 2s and 2s+1, so S, X and U feed the B operand from
// registers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x8 frag(const u32x4* base, int f, int lane) {
    return __builtin_bit_cast(bf16x8, base[64 * f + lane]);
}
// T / M fragment f (half fragments carry zero values 4..7)
__device__ __forceinline__ bf16x8 frag_tm(const u32x4* mat, int f, int lane) {
    if (tm_half(f)) {
        const uint2 x = reinterpret_cast<const uint2*>(mat + tm_off(f) / 16)[lane];
        return __builtin_bit_cast(bf16x8, u32x4{x.x, x.y, 0u, 0u});
    }
    return __builtin_bit_cast(bf16x8, mat[tm_off(f) / 16 + lane]);
}

// CONV: v holds the raw values before the short convolution, which the
// loaders apply to each V piece before it goes to LDS (rounded to bf16).
template <bool CONV>
__global__ __launch_bounds__(512, 1) void kda_scan16_kernel(
    const uint8_t* __restrict__ ws, const uint16_t* __restrict__ v, float scale,
    const float* h_in, float* h_out, uint16_t* __restrict__ out, int T, int H, int chunk0,
    int nchunks, ConvArgs conv, WaitCtl wait) {
    // The record, verbatim: Kt / Qt once, the rest (Kb^T, T / M, gamma) in two
    // buffers by chunk parity, so that the rest of chunk i + 1 is in place
    // while chunk i is scanned.
    constexpr int kRest = (Rec16::BYTES - Rec16::KB) / 16;  // pieces
    __shared__ u32x4 kq_s[Rec16::KB / 16];
    __shared__ u32x4 rest_s[2][kRest];
    __shared__ __align__(16) uint16_t v_s[kChunk * VP];    // V slice, [token][column]
    // Kt/Qt/V ready; Kt/Qt/V consumed; rest ready (per buffer, 2); abort;
    // output stored; rest consumed (per buffer, 2).  The double-buffered rest
    // needs a counter per buffer: waves of a role may be a chunk apart, and a
    // shared counter would let one wave's signal for the later chunk stand in
    // for another's for the earlier one.  The single Kt / Qt / V buffer keeps
    // the roles in step by itself.
    __shared__ unsigned sync_s[8];

    // Workgroups are dealt round-robin to the 8 XCDs (each with its own L2):
    // both slices of a head go to one XCD, so the records that both read come
    // from HBM once.
    const int BH = gridDim.x / kSlices;  // records are stored chunk-major
    int slice, bh;
    {
        const int nblk = gridDim.x, id = blockIdx.x;
        if (nblk % (8 * kSlices) == 0) {
            const int per_xcd = nblk / 8, xcd = id % 8, idx = id / 8;
            bh = xcd * (per_xcd / kSlices) + idx / kSlices;
            slice = idx % kSlices;
        } else {
            slice = id % kSlices;
            bh = id / kSlices;
        }
    }
    const int h = bh % H, b = bh / H;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;

    if (tid < 8) sync_s[tid] = 0u;
    __syncthreads();  // the only workgroup barrier: roles split below

    if (wv < 4) {
        // =====================================================================
        // loaders: 16-byte pieces tid + 256 m of each record part, one chunk
        // ahead in registers
        // =====================================================================
        // V of the slice: 64 tokens x 64 columns = 512 pieces of 8 columns, two
        // per thread (piece tid + 256 m: token piece >> 3, columns 8 (piece & 7))
        u32x4 ra[8], rb[kRestFull + 1], rv[2];
        const int64_t vstride = (int64_t)H * kD;
        const uint16_t* vslice = v + ((int64_t)b * T * H + h) * kD + kCols * slice;
        // short convolution of V: a wave's piece m holds 8 consecutive tokens
        // (lane L: token L / 8, columns 8 (L % 8)), so the 3 tokens before a
        // lane's token sit 8, 16, 24 lanes down; lanes of tokens 5..7 also
        // load the rows 8 tokens back (rh), which the shifts hand to the
        // lanes of tokens 0..2.  The taps of this thread's 8 columns are the
        // same for both pieces; the state rows of the slice are tokens -3..-1.
        u32x4 rh[2];
        f32x4 wcol[8];
        const uint16_t* vst = nullptr;
        if constexpr (CONV) {
            const float* wr = conv.wv + ((size_t)h * kD + kCols * slice + (tid & 7) * 8) * 4;
#pragma unroll
            for (int e = 0; e < 8; ++e) wcol[e] = *reinterpret_cast<const f32x4*>(wr + 4 * e);
            if (conv.state)
                vst = conv.state + (size_t)2 * conv.B * 3 * H * kD +
                      ((int64_t)b * 3 * H + h) * kD + kCols * slice;
        }
#define KDA_LOAD_ISSUE(cl_)                                                                      \
    do {                                                                                         \
        const u32x4* src_ = reinterpret_cast<const u32x4*>(                                      \
            ws + ((size_t)(cl_) * BH + bh) * Rec16::BYTES);                                      \
        _Pragma("unroll") for (int m_ = 0; m_ < 8; ++m_) ra[m_] = src_[tid + 256 * m_];          \
        _Pragma("unroll") for (int m_ = 0; m_ < kRestFull; ++m_)                                \
            rb[m_] = src_[2048 + tid + 256 * m_];                                                \
        rb[kRestFull] = src_[2048 + 256 * kRestFull + (tid < kRestTail ? tid : 0)];              \
        _Pragma("unroll") for (int m_ = 0; m_ < 2; ++m_) {                                       \
            const int pc_ = tid + 256 * m_;                                                      \
            const int64_t tk_ = (int64_t)(chunk0 + (cl_)) * kChunk + (pc_ >> 3);                 \
            rv[m_] = *reinterpret_cast<const u32x4*>(vslice + (tk_ < T ? tk_ : 0) * vstride +     \
                                                     (pc_ & 7) * 8);                             \
            if constexpr (CONV) {                                                                \
                /* token 8 back, for lanes of tokens 5..7: >= -3, and only the */                \
                /* first piece of a sequence reaches before it; a clamped */                     \
                /* address where the value is unused, zeroed at use */                           \
                if ((pc_ >> 3) % 8 >= 5) {                                                       \
                    const int64_t t_ = tk_ - 8;                                                  \
                    const uint16_t* src_ =                                                       \
                        t_ >= 0 ? vslice + (t_ < T ? t_ : T - 1) * vstride + (pc_ & 7) * 8       \
                        : vst   ? vst + (3 + t_) * vstride + (pc_ & 7) * 8                       \
                                : vslice + (pc_ & 7) * 8;                                        \
                    rh[m_] = *reinterpret_cast<const u32x4*>(src_);                              \
                }                                                                                \
            }                                                                                    \
        }                                                                                        \
    } while (0)
        // Per chunk i: the rest into buffer i & 1 (released by chunk i - 2),
        // Kt / Qt / V once chunk i - 1 has multiplied them, and the loads of
        // chunk i + 1 once the output of chunk i - 1 is stored: the burst of
        // loads then runs beside the state update of chunk i - 1 and the
        // products of chunk i, which touch no global memory (loads issued
        // beside the output stores hold those up).
        KDA_LOAD_ISSUE(0);
        for (int i = 0; i < nchunks; ++i) {
            wait_for(&sync_s[6 + (i & 1)], 4u * (unsigned)(i >> 1), &sync_s[4], wait.spin_limit);
            u32x4* rs = rest_s[i & 1];
#pragma unroll
            for (int m = 0; m < kRestFull; ++m) rs[tid + 256 * m] = rb[m];
            if (tid < kRestTail) rs[tid + 256 * kRestFull] = rb[kRestFull];
            signal(&sync_s[2 + (i & 1)], lane);
            // V of the chunk, filtered before the wait below so that the
            // filter does not hold up the scan waves; tokens past the end of
            // the sequence have zero V
            u32x4 vx[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int pc = tid + 256 * m, tk = pc >> 3;
                const int64_t tkg = (int64_t)(chunk0 + i) * kChunk + tk;
                const bool ok = tkg < T;
                u32x4 x = rv[m];
                if constexpr (CONV) {
                    // silu(sum_j w_j v_{t-3+j}) per column, taps before the
                    // sequence from the state or zero.  xj[j]: token t - 3 + j,
                    // from lane L - 8 (3 - j) of the own rows, or, across the
                    // piece's start, of the back rows
                    const int u = lane >> 3;
                    const bool zero_back = tkg - 8 < 0 && vst == nullptr;
                    u32x4 back = rh[m];
                    if (zero_back) back = u32x4{0u, 0u, 0u, 0u};
                    u32x4 xj[4];
                    xj[3] = x;
#pragma unroll
                    for (int d = 1; d <= 3; ++d) {
                        const int from = ((lane - 8 * d) & 63) << 2;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            xj[3 - d][e] = (uint32_t)__builtin_amdgcn_ds_bpermute(
                                from, (int)(u + d >= 8 ? back[e] : x[e]));
                    }
                    float y[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float acc = 0.f;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t wd = xj[j][e >> 1];
                            const float xv =
                                __builtin_bit_cast(float, (e & 1) ? (wd & 0xffff0000u) : (wd << 16));
                            acc += wcol[e][j] * xv;
                        }
                        y[e] = acc * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * acc));
                    }
                    x = u32x4{pack2(y[0], y[1]), pack2(y[2], y[3]), pack2(y[4], y[5]),
                              pack2(y[6], y[7])};
                }
                vx[m] = ok ? x : u32x4{0u, 0u, 0u, 0u};
            }
            // Kt, Qt (pieces 0..2047) and V, once the scan waves are done
            // with the previous ones
            wait_for(&sync_s[1], 4u * i, &sync_s[4], wait.spin_limit);
#pragma unroll
            for (int m = 0; m < 8; ++m) kq_s[tid + 256 * m] = ra[m];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int pc = tid + 256 * m, tk = pc >> 3;
                uint2* d2 = reinterpret_cast<uint2*>(&v_s[tk * VP + (pc & 7) * 8]);
                d2[0] = uint2{vx[m][0], vx[m][1]};
                d2[1] = uint2{vx[m][2], vx[m][3]};
            }
            signal(&sync_s[0], lane);
            if (i + 1 < nchunks) {
                wait_for(&sync_s[5], 4u * i, &sync_s[4], wait.spin_limit);
                KDA_LOAD_ISSUE(i + 1);
            }
        }
#undef KDA_LOAD_ISSUE
    } else {
        // =====================================================================
        // scan waves: they carry the serial chain, so they win issue over the
        // loader wave that shares their SIMD
        // =====================================================================
        __builtin_amdgcn_s_setprio(3);
        const int w = wv - 4;
        const int j0 = kCols * slice + 16 * w;
        const u32x4* kt_s = kq_s + Rec16::KT / 16;
        const u32x4* qt_s = kq_s + Rec16::QT / 16;
        // V to accumulator layout on the matrix cores: fragment rows are tokens,
        // k the 32 columns 32 (w / 2) ..; the 0/1 selection B (value e of lane
        // (j, gq) is 1 where its column is 16 (w & 1) + j) returns lane (j, g)
        // the tokens 16rt + 4g .. +3 of column 16w + j, exactly.
        bf16x8 selv;
        {
            u32x4 u;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int e0 = 2 * x, e1 = 2 * x + 1;
                const int c0 = (e0 < 4 ? 4 * gq + e0 : 16 + 4 * gq + e0 - 4);
                const int c1 = (e1 < 4 ? 4 * gq + e1 : 16 + 4 * gq + e1 - 4);
                u[x] = (c0 == 16 * (w & 1) + n ? 0x3f80u : 0u) |
                       (c1 == 16 * (w & 1) + n ? 0x3f800000u : 0u);
            }
            selv = __builtin_bit_cast(bf16x8, u);
        }
        f32x4 S[8];
        const float* hin = h_in ? h_in + (size_t)bh * kD * kD : nullptr;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[t][e] = hin ? hin[(size_t)(16 * t + 4 * gq + e) * kD + j0 + n] : 0.f;

        const int64_t rstride = (int64_t)H * kD;  // elements between tokens

        // The output gate, off the chain from one state to the next: the
        // logits of this lane's outputs (token 16 rt + n, columns j0 + 4 gq
        // ..) are loaded a chunk ahead (zr) and turned into sigmoids (sg)
        // beside the previous chunk's state-update products.
        const uint16_t* gate = CONV ? conv.gate : nullptr;
        const uint16_t* gatec = gate ? gate + ((int64_t)b * T * H + h) * kD + j0 + 4 * gq : nullptr;
        uint2 zr[4];
        f32x4 sg[4];
        auto gate_load = [&](int ci) {  // logits of local chunk ci (clamped rows)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int64_t tk = (int64_t)(chunk0 + ci) * kChunk + 16 * rt + n;
                zr[rt] = *reinterpret_cast<const uint2*>(gatec + (tk < T ? tk : T - 1) * rstride);
            }
        };
        auto gate_sigmoid = [&]() {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const float z[4] = {bf2f((uint16_t)zr[rt].x), bf2f((uint16_t)(zr[rt].x >> 16)),
                                    bf2f((uint16_t)zr[rt].y), bf2f((uint16_t)(zr[rt].y >> 16))};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sg[rt][e] = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * z[e]));
            }
        };
        if (gatec) {
            gate_load(0);
            gate_sigmoid();
            gate_load(1);
        }
        for (int i = 0; i < nchunks; ++i) {
            const int64_t c0 = (int64_t)(chunk0 + i) * kChunk;
            wait_for(&sync_s[0], 4u * (i + 1), &sync_s[4], wait.spin_limit);

            // Pk = Kt S (rows token 4g + e, column n) and Pq = (Qt S)^T (rows
            // column 4g + e, column token n): the S slice serves as the B
            // operand of the first and, transposed, as the A operand of the
            // second, with the same registers
            // (fragments of k-step s + 1 are read while step s multiplies)
            f32x4 Pk[4], Pq[4], Vt[4];
            bf16x8 fv[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                Pk[rt] = Pq[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
                fv[rt] = frag_row(v_s, VP, 16 * rt + n, 32 * (w >> 1), gq);
            }
            bf16x8 fk[2][4], fq[2][4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                fk[0][rt] = frag(kt_s, 4 * rt, lane);
                fq[0][rt] = frag(qt_s, 4 * rt, lane);
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) Vt[rt] = mma(f32x4{0.f, 0.f, 0.f, 0.f}, fv[rt], selv);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s < 3) {
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) {
                        fk[(s + 1) & 1][rt] = frag(kt_s, 4 * rt + s + 1, lane);
                        fq[(s + 1) & 1][rt] = frag(qt_s, 4 * rt + s + 1, lane);
                    }
                }
                // keep these reads ahead of this step's products
                __builtin_amdgcn_sched_barrier(0);
                const bf16x8 bS = pack_b(S[2 * s], S[2 * s + 1]);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    Pk[rt] = mma(Pk[rt], fk[s & 1][rt], bS);
                    Pq[rt] = mma(Pq[rt], bS, fq[s & 1][rt]);
                }
            }
            signal(&sync_s[1], lane);  // Kt, Qt, V consumed
            wait_for(&sync_s[2 + (i & 1)], 4u * (unsigned)((i >> 1) + 1), &sync_s[4], wait.spin_limit);
            const u32x4* rs = rest_s[i & 1];
            const u32x4* kb_s = rs;
            const u32x4* th_s = rs + (Rec16::TM - Rec16::KB + 0 * Rec16::kTM) / 16;
            const u32x4* tl_s = rs + (Rec16::TM - Rec16::KB + 1 * Rec16::kTM) / 16;
            const u32x4* mh_s = rs + (Rec16::TM - Rec16::KB + 2 * Rec16::kTM) / 16;
            const float* gam_s = reinterpret_cast<const float*>(rs + (Rec16::G - Rec16::KB) / 16);

            // U = T (V - Kt S), both factors as hi + lo (T lower triangular);
            // the six T fragment pairs are read before X is split
            bf16x8 fth[6], ftl[6];
#pragma unroll
            for (int f = 0; f < 6; ++f) {
                fth[f] = frag_tm(th_s, f, lane);
                ftl[f] = frag_tm(tl_s, f, lane);
            }
            __builtin_amdgcn_sched_barrier(0);
            bf16x8 bh_[2], bl_[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                split_b(Vt[2 * s2] - Pk[2 * s2], Vt[2 * s2 + 1] - Pk[2 * s2 + 1], bh_[s2], bl_[s2]);
            f32x4 U[4];
#pragma unroll
            for (int f = 0; f < 6; ++f) {
                const int rt = tm_rt(f), s2 = tm_s2(f);
                if (s2 == 0) U[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
                U[rt] = mma(U[rt], fth[f], bh_[s2]);
                U[rt] = mma(U[rt], ftl[f], bh_[s2]);
                U[rt] = mma(U[rt], fth[f], bl_[s2]);
            }
            // the M fragments (same six positions) are read while U is split
            bf16x8 fmh[6];
#pragma unroll
            for (int f = 0; f < 6; ++f) {
                fmh[f] = frag_tm(mh_s, f, lane);
            }
            __builtin_amdgcn_sched_barrier(0);

            // O^T = (Qt S)^T + U^T M^T (U as hi + lo, M bf16), so that a lane
            // holds token 16rt + n and the four consecutive columns j0 + 4g ..
            // +3; then S <- Diag(gamma) S + Kb^T U (U as hi + lo).  This order
            // (output, then state update) measured faster than the reverse.
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) split_b(U[2 * s2], U[2 * s2 + 1], bh_[s2], bl_[s2]);
            // after the swap below, lane (n, g) holds token 16 rt + n of tile
            // rt = 2 pr + (g & 1) and the eight columns j0 + 8 (g / 2) ..
            uint16_t* outc = out + ((int64_t)b * T * H + h) * kD + j0 + 8 * (gq >> 1);
            // Kb^T fragments of the first half of the state rows
            bf16x8 fkb[2][4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) fkb[0][t][s2] = frag(kb_s, 2 * t + s2, lane);
            __builtin_amdgcn_sched_barrier(0);
            uint32_t ob[4][2];  // bf16 outputs per tile: columns 4g .. +1, +2 .. +3
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 o = Pq[rt];
#pragma unroll
                for (int f = 0; f < 6; ++f) {
                    if (tm_rt(f) != rt) continue;
                    const int s2 = tm_s2(f);
                    o = mma(o, bh_[s2], fmh[f]);
                    o = mma(o, bl_[s2], fmh[f]);
                }
                f32x4 y = scale * o;
                if (gatec) y *= sg[rt];  // out = o * sigmoid(z)
                ob[rt][0] = pack2(y[0], y[1]);
                ob[rt][1] = pack2(y[2], y[3]);
            }
            // Tiles 2 pr and 2 pr + 1: a swap of the odd 16-lane rows of one
            // register with the even rows of another hands the even rows (g =
            // 0, 2) columns 8 (g / 2) .. +7 of the first tile and the odd rows
            // the same columns of the second, one 16-byte store per lane.
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const auto a = __builtin_amdgcn_permlane16_swap(ob[2 * pr][0], ob[2 * pr + 1][0], false, false);
                const auto c = __builtin_amdgcn_permlane16_swap(ob[2 * pr][1], ob[2 * pr + 1][1], false, false);
                const int64_t tk = c0 + 16 * (2 * pr + (gq & 1)) + n;
                if (tk < T)
                    *reinterpret_cast<u32x4*>(outc + tk * rstride) = u32x4{a[0], c[0], a[1], c[1]};
            }
            signal(&sync_s[5], lane);  // the output is stored
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                if (half == 0) {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2)
                            fkb[1][t][s2] = frag(kb_s, 2 * (t + 4) + s2, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    // the next chunk's gate beside these products; then the
                    // logits of the one after
                    if (gatec) {
                        gate_sigmoid();
                        gate_load(i + 2);
                    }
                }
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) {
                    const int t = 4 * half + t4;
                    const f32x4 gm = *reinterpret_cast<const f32x4*>(&gam_s[16 * t + 4 * gq]);
                    S[t] *= gm;
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        S[t] = mma(S[t], fkb[half][t4][s2], bh_[s2]);
                        S[t] = mma(S[t], fkb[half][t4][s2], bl_[s2]);
                    }
                }
            }
            signal(&sync_s[6 + (i & 1)], lane);  // the rest consumed
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
        __hip_atomic_load(&sync_s[4], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0u)
        wait.abort_out[0] = 1u;
}

hipError_t launch_prep16(const void* q, const void* k, const void* g, bool g_bf16,
                         const float* beta, int B, int T, int H, int chunk0, int nchunks, void* ws,
                         const ConvArgs& conv, hipStream_t stream) {
    const unsigned nblk = (unsigned)((int64_t)B * H * nchunks);
    const uint16_t* q16 = static_cast<const uint16_t*>(q);
    const uint16_t* k16 = static_cast<const uint16_t*>(k);
    uint8_t* w8 = static_cast<uint8_t*>(ws);
    const bool cv = conv.wq != nullptr;
    if (g_bf16 && cv)
        hipLaunchKernelGGL((kda_prep16_kernel<true, true>), dim3(nblk), dim3(256), 0, stream,
                           q16, k16, g, beta, T, H, chunk0, nchunks, w8, conv);
    else if (g_bf16)
        hipLaunchKernelGGL((kda_prep16_kernel<true, false>), dim3(nblk), dim3(256), 0, stream,
                           q16, k16, g, beta, T, H, chunk0, nchunks, w8, conv);
    else if (cv)
        hipLaunchKernelGGL((kda_prep16_kernel<false, true>), dim3(nblk), dim3(256), 0, stream,
                           q16, k16, g, beta, T, H, chunk0, nchunks, w8, conv);
    else
        hipLaunchKernelGGL((kda_prep16_kernel<false, false>), dim3(nblk), dim3(256), 0, stream,
                           q16, k16, g, beta, T, H, chunk0, nchunks, w8, conv);
    return hipGetLastError();
}

hipError_t launch_scan16(const void* ws, const void* v, const float* h_in, float* h_out,
                         void* out, float scale, int B, int T, int H, int chunk0, int nchunks,
                         const ConvArgs& conv, const WaitCtl& wait, hipStream_t stream) {
    const unsigned nblk = (unsigned)((int64_t)B * H * kSlices);
    if (conv.wq)
        hipLaunchKernelGGL(kda_scan16_kernel<true>, dim3(nblk), dim3(512), 0, stream,
                           static_cast<const uint8_t*>(ws), static_cast<const uint16_t*>(v), scale,
                           h_in, h_out, static_cast<uint16_t*>(out), T, H, chunk0, nchunks, conv,
                           wait);
    else
        hipLaunchKernelGGL(kda_scan16_kernel<false>, dim3(nblk), dim3(512), 0, stream,
                           static_cast<const uint8_t*>(ws), static_cast<const uint16_t*>(v), scale,
                           h_in, h_out, static_cast<uint16_t*>(out), T, H, chunk0, nchunks, conv,
                           wait);
    return hipGetLastError();
}

// one thread per (tensor, batch, head, channel): its 3 values are read before
// any is written, so st_out may equal conv.state
__global__ void kda_conv_state_out_kernel(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                          int B, int T, int H, const uint16_t* st_in,
                                          uint16_t* st_out) {
    const int64_t n = (int64_t)3 * B * H * kD;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(idx % kD);
        const int h = (int)((idx / kD) % H);
        const int b = (int)((idx / ((int64_t)kD * H)) % B);
        const int ten = (int)(idx / ((int64_t)kD * H * B));
        const uint16_t* x = ten == 0 ? q : ten == 1 ? k : v;
        uint16_t val[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int64_t t = (int64_t)T - 3 + j;
            val[j] = t >= 0 ? x[(((int64_t)b * T + t) * H + h) * kD + c]
                   : st_in ? st_in[((((int64_t)ten * B + b) * 3 + (3 + t)) * H + h) * kD + c]
                           : (uint16_t)0;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) st_out[((((int64_t)ten * B + b) * 3 + j) * H + h) * kD + c] = val[j];
    }
}

hipError_t launch_conv_state_out(const void* q, const void* k, const void* v, int B, int T,
                                 int H, const ConvArgs& conv, void* st_out, hipStream_t stream) {
    const int64_t n = (int64_t)3 * B * H * kD;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(kda_conv_state_out_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), B, T, H, conv.state,
                       static_cast<uint16_t*>(st_out));
    return hipGetLastError();
}

}  // namespace kda
