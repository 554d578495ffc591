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
//   prep  (kda_chunk.hip) writes each chunk's record (W, Q', Kb^T, T, M T,
//         gamma) and X = (I + A)^-1;
//   state scan    walks the chunks forward and stores the state entering each;
//   gradient scan walks them in reverse and stores dS' of each chunk, and dS
//         of the first as the initial state's gradient;
//   chunk gradients, one workgroup per (batch, head, chunk), rebuilds the
//         chunk's matrices from q, k, g, beta and writes dq, dk, dv, dg, dbeta.
// Every product runs on the fp32 matrix cores (v_mfma_f32_16x16x4_f32) with
// its operands in LDS or registers.
#include <type_traits>

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

// C[M][N] = sum_k A(i, k) B(k, j) on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32).  The operand functors return four values along k:
// A4(i, k) = A(i, k .. k + 3), B4(k, j) = B(k .. k + 3, j).  The result is
// cut into 16 x 16 tiles; wave w takes column tile w mod (N / 16) and every
// (NT / 64) / (N / 16)-th row tile from w / (N / 16) on, so the B operand it
// loads serves all its tiles and their loads are in flight together.  For a
// tile at (i0, j0), lane (n = lane % 16, g = lane / 16) loads A(i0 + n, k0 +
// 4g .. + 3) and B(k0 + 4g .. + 3, j0 + n); MFMA e of a 16-wide k block takes
// value e of each, so lane (n, g) stands for k = k0 + 4g + e in both operands.
// The accumulator holds C[i0 + 4g + e][j0 + n], handed to out(i, j, value).
// K is a multiple of 16.
template <int M, int N, int NT, class FA, class FB, class FO>
__device__ __forceinline__ void mmf(int K, FA&& A4, FB&& B4, FO&& out) {
    constexpr int TR = M / 16, TC = N / 16, W = NT / 64;
    static_assert(M % 16 == 0 && N % 16 == 0 && NT % 64 == 0, "16 x 16 tiles, whole waves");
    static_assert(W % TC == 0 && (TR * TC) % W == 0, "each wave keeps one column tile");
    constexpr int RPW = TR * TC / W;  // row tiles per wave
    constexpr int RSTEP = W / TC;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int j0 = 16 * (w % TC), r0 = w / TC;
    f32x4 acc[RPW];
#pragma unroll
    for (int u = 0; u < RPW; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int k0 = 0; k0 < K; k0 += 16) {
        const float4 b = B4(k0 + 4 * g, j0 + n);
        float4 a[RPW];
#pragma unroll
        for (int u = 0; u < RPW; ++u) a[u] = A4(16 * (r0 + RSTEP * u) + n, k0 + 4 * g);
#pragma unroll
        for (int u = 0; u < RPW; ++u) {
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u].x, b.x, acc[u], 0, 0, 0);
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u].y, b.y, acc[u], 0, 0, 0);
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u].z, b.z, acc[u], 0, 0, 0);
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u].w, b.w, acc[u], 0, 0, 0);
        }
    }
#pragma unroll
    for (int u = 0; u < RPW; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * (r0 + RSTEP * u) + 4 * g + e;
            // out(m, i, j, v) also gets the element's slot m = 4 u + e in the lane
            if constexpr (std::is_invocable_v<FO, int, int, int, float>)
                out(4 * u + e, i, j0 + n, acc[u][e]);
            else
                out(i, j0 + n, acc[u][e]);
        }
}

__device__ __forceinline__ float4 ld4(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
// four values down a column of a row-major matrix
__device__ __forceinline__ float4 col4(const float* p, size_t pitch) {
    return make_float4(p[0], p[pitch], p[2 * pitch], p[3 * pitch]);
}
// q / k / v / dout in and dq / dk / dv out: fp32, or bf16 widened on load and
// rounded to nearest even on store (8-byte aligned groups of four)
__device__ __forceinline__ float io1(const float* p) { return *p; }
__device__ __forceinline__ float io1(const uint16_t* p) { return bf2f(*p); }
__device__ __forceinline__ float4 io4(const float* p) { return ld4(p); }
__device__ __forceinline__ float4 io4(const uint16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__builtin_bit_cast(float, u.x << 16),
                       __builtin_bit_cast(float, u.x & 0xffff0000u),
                       __builtin_bit_cast(float, u.y << 16),
                       __builtin_bit_cast(float, u.y & 0xffff0000u));
}
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

// LDS row pitches of the staged record parts: four floats of padding per row,
// so rows stay 16-byte aligned (float4 reads and writes) while the rows that a
// wave reads at one k fall in different banks
constexpr int kP64 = kChunk + 4;
constexpr int kP128 = kD + 4;

// ---------------------------------------------------------------------------
// State scan: one workgroup per (b, h, 64 value columns).  For chunk c the
// state slice entering it is stored, then S <- Diag(gamma) S + Kb^T (T V - W S).
// Each chunk's record parts and V slice are first staged in LDS.
// ---------------------------------------------------------------------------
struct __align__(16) StateScanLds {
    float S[kD][kScanCols];
    float Z[kChunk][kScanCols];
    float Tm[kChunk * kP64];
    float W[kChunk * kP128];
    float KT[kD * kP64];
    float V[kChunk][kScanCols];
    float gam[kD];
};

// Chunks chunk0 .. chunk0 + nch - 1 of the sequence (records, states local to
// the segment); h_out (or NULL) receives the state leaving the last one.
template <typename IO>
__global__ __launch_bounds__(kScanThreads, 1) void kda_bwd_state_scan_kernel(
    const uint8_t* __restrict__ rec, const IO* __restrict__ v, const float* __restrict__ h0,
    float* __restrict__ states, float* __restrict__ h_out, int T, int H, int chunk0, int nch) {
    __shared__ StateScanLds s;
    int bh, slice;
    scan_ids(bh, slice);
    const int b = bh / H, h = bh % H;
    const int col0 = slice * kScanCols;
    const int tid = threadIdx.x;
    for (int e = tid; e < kD * kScanCols; e += kScanThreads) {
        const int i = e / kScanCols, j = e % kScanCols;
        s.S[i][j] = h0 ? h0[(size_t)bh * kStateFloats + (size_t)i * kD + col0 + j] : 0.f;
    }
    // The next chunk's record parts and V slice are loaded into registers while
    // the current chunk computes: float4 number tid + 512 u of T (u < 2), W
    // (u < 6), Kb^T (u < 10) and V (u < 12).
    static_assert(kScanThreads == 512 && kScanCols == 64, "prefetch layout");
    float4 pf[12];
    float gpf = 0.f;
    auto fetch = [&](int c) {
        const uint8_t* r = rec + ((size_t)bh * nch + c) * RF::BYTES;
        const int cg = chunk0 + c;
        const int L = min(kChunk, T - cg * kChunk);
        const float* Tg = reinterpret_cast<const float*>(r + RF::TH);
        const float* Wg = reinterpret_cast<const float*>(r + RF::W);
        const float* Kg = reinterpret_cast<const float*>(r + RF::KT);
        const IO* Vg = v + (((size_t)b * T + (size_t)cg * kChunk) * H + h) * kD + col0;
#pragma unroll
        for (int u = 0; u < 12; ++u) {
            if (u < 2) {
                const int e = tid + 512 * u;
                pf[u] = ld4(Tg + (e >> 4) * kChunk + 4 * (e & 15));
            } else if (u < 6) {
                const int e = tid + 512 * (u - 2);
                pf[u] = ld4(Wg + (e >> 5) * kD + 4 * (e & 31));
            } else if (u < 10) {
                const int e = tid + 512 * (u - 6);
                pf[u] = ld4(Kg + (e >> 4) * kChunk + 4 * (e & 15));
            } else {
                const int e = tid + 512 * (u - 10), row = e >> 4;
                pf[u] = row < L ? io4(Vg + (size_t)row * H * kD + 4 * (e & 15))
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        if (tid < kD) gpf = reinterpret_cast<const float*>(r + RF::G)[tid];
    };
    auto put = [&]() {
#pragma unroll
        for (int u = 0; u < 12; ++u) {
            float* d;
            if (u < 2) {
                const int e = tid + 512 * u;
                d = &s.Tm[(e >> 4) * kP64 + 4 * (e & 15)];
            } else if (u < 6) {
                const int e = tid + 512 * (u - 2);
                d = &s.W[(e >> 5) * kP128 + 4 * (e & 31)];
            } else if (u < 10) {
                const int e = tid + 512 * (u - 6);
                d = &s.KT[(e >> 4) * kP64 + 4 * (e & 15)];
            } else {
                const int e = tid + 512 * (u - 10);
                d = &s.V[e >> 4][4 * (e & 15)];
            }
            *reinterpret_cast<float4*>(d) = pf[u];
        }
        if (tid < kD) s.gam[tid] = gpf;
    };
    fetch(0);
    for (int c = 0; c < nch; ++c) {
        __syncthreads();  // the previous chunk's reads of the staged parts are done
        put();
        float* st = states + ((size_t)bh * nch + c) * kStateFloats;
        for (int e = tid; e < kD * kScanCols; e += kScanThreads) {
            const int i = e / kScanCols, j = e % kScanCols;
            st[(size_t)i * kD + col0 + j] = s.S[i][j];
        }
        __syncthreads();
        if (c + 1 < nch) fetch(c + 1);
        // Z = T V - W S
        mmf<kChunk, kScanCols, kScanThreads>(
            kChunk + kD,
            [&](int i, int k) {
                return k < kChunk ? ld4(&s.Tm[i * kP64 + k])
                                  : scale4(ld4(&s.W[i * kP128 + (k - kChunk)]), -1.f);
            },
            [&](int k, int j) {
                return k < kChunk ? col4(&s.V[k][j], kScanCols) : col4(&s.S[k - kChunk][j], kScanCols);
            },
            [&](int i, int j, float a) { s.Z[i][j] = a; });
        __syncthreads();
        // S' = Diag(gamma) S + Kb^T Z (each lane updates only its own entries)
        mmf<kD, kScanCols, kScanThreads>(
            kChunk, [&](int i, int k) { return ld4(&s.KT[i * kP64 + k]); },
            [&](int k, int j) { return col4(&s.Z[k][j], kScanCols); },
            [&](int i, int j, float a) { s.S[i][j] = fmaf(s.gam[i], s.S[i][j], a); });
    }
    if (h_out) {
        __syncthreads();
        for (int e = tid; e < kD * kScanCols; e += kScanThreads) {
            const int i = e / kScanCols, j = e % kScanCols;
            h_out[(size_t)bh * kStateFloats + (size_t)i * kD + col0 + j] = s.S[i][j];
        }
    }
}

// ---------------------------------------------------------------------------
// Gradient scan: chunks in reverse.  For chunk c, dS' (the gradient of the
// state leaving it) is stored, then
//   dS <- Diag(gamma) dS' - W^T (Kb dS') + scale Q'^T dO.
// After chunk 0, dS is the initial state's gradient.  Kb^T and then W take
// turns in one LDS buffer.
// ---------------------------------------------------------------------------
struct __align__(16) GradScanLds {
    float D[kD][kScanCols];
    float Y[kChunk][kScanCols];
    float KW[kD * kP64];  // Kb^T [128][64], then W [64][128] (at pitch kP128 it fits)
    float QP[kChunk * kP128];
    float O[kChunk][kScanCols];
    float gam[kD];
};
static_assert(kD * kP64 >= kChunk * kP128, "W must fit in the Kb^T buffer");

// Chunks chunk0 .. chunk0 + nch - 1 (records and dS' local to the segment):
// dhT is the gradient of the state leaving the last of them, dh0 receives that
// of the state entering the first.  dh0 may equal dhT (each workgroup reads its
// slice before it writes it).
template <typename IO>
__global__ __launch_bounds__(kScanThreads, 1) void kda_bwd_grad_scan_kernel(
    const uint8_t* __restrict__ rec, const IO* __restrict__ dout, const float* dhT,
    float* __restrict__ dsn, float* dh0, float scale, int T, int H, int chunk0, int nch) {
    __shared__ GradScanLds s;
    int bh, slice;
    scan_ids(bh, slice);
    const int b = bh / H, h = bh % H;
    const int col0 = slice * kScanCols;
    const int tid = threadIdx.x;
    for (int e = tid; e < kD * kScanCols; e += kScanThreads) {
        const int i = e / kScanCols, j = e % kScanCols;
        s.D[i][j] = dhT ? dhT[(size_t)bh * kStateFloats + (size_t)i * kD + col0 + j] : 0.f;
    }
    // The next chunk's record parts and dO slice are loaded into registers while
    // the current chunk computes: float4 number tid + 512 u of Kb^T (u < 4),
    // Q' (u < 8), dO (u < 10) and W (u < 14).
    static_assert(kScanThreads == 512 && kScanCols == 64, "prefetch layout");
    float4 pf[14];
    float gpf = 0.f;
    auto fetch = [&](int c) {
        const uint8_t* r = rec + ((size_t)bh * nch + c) * RF::BYTES;
        const int cg = chunk0 + c;
        const int L = min(kChunk, T - cg * kChunk);
        const float* Kg = reinterpret_cast<const float*>(r + RF::KT);
        const float* Qg = reinterpret_cast<const float*>(r + RF::QP);
        const float* Wg = reinterpret_cast<const float*>(r + RF::W);
        const IO* Og = dout + (((size_t)b * T + (size_t)cg * kChunk) * H + h) * kD + col0;
#pragma unroll
        for (int u = 0; u < 14; ++u) {
            if (u < 4) {
                const int e = tid + 512 * u;
                pf[u] = ld4(Kg + (e >> 4) * kChunk + 4 * (e & 15));
            } else if (u < 8) {
                const int e = tid + 512 * (u - 4);
                pf[u] = ld4(Qg + (e >> 5) * kD + 4 * (e & 31));
            } else if (u < 10) {
                const int e = tid + 512 * (u - 8), row = e >> 4;
                pf[u] = row < L ? io4(Og + (size_t)row * H * kD + 4 * (e & 15))
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            } else {
                const int e = tid + 512 * (u - 10);
                pf[u] = ld4(Wg + (e >> 5) * kD + 4 * (e & 31));
            }
        }
        if (tid < kD) gpf = reinterpret_cast<const float*>(r + RF::G)[tid];
    };
    auto put4 = [&](float* d, float4 x) { *reinterpret_cast<float4*>(d) = x; };
    auto put = [&]() {  // Kb^T, Q', dO and gamma
#pragma unroll
        for (int u = 0; u < 10; ++u) {
            if (u < 4) {
                const int e = tid + 512 * u;
                put4(&s.KW[(e >> 4) * kP64 + 4 * (e & 15)], pf[u]);
            } else if (u < 8) {
                const int e = tid + 512 * (u - 4);
                put4(&s.QP[(e >> 5) * kP128 + 4 * (e & 31)], pf[u]);
            } else {
                const int e = tid + 512 * (u - 8);
                put4(&s.O[e >> 4][4 * (e & 15)], pf[u]);
            }
        }
        if (tid < kD) s.gam[tid] = gpf;
    };
    auto put_w = [&]() {  // W, over Kb^T
#pragma unroll
        for (int u = 10; u < 14; ++u) {
            const int e = tid + 512 * (u - 10);
            put4(&s.KW[(e >> 5) * kP128 + 4 * (e & 31)], pf[u]);
        }
    };
    fetch(nch - 1);
    for (int c = nch - 1; c >= 0; --c) {
        __syncthreads();  // the previous chunk's reads of the staged parts are done
        put();
        float* st = dsn + ((size_t)bh * nch + c) * kStateFloats;
        for (int e = tid; e < kD * kScanCols; e += kScanThreads) {
            const int i = e / kScanCols, j = e % kScanCols;
            st[(size_t)i * kD + col0 + j] = s.D[i][j];
        }
        __syncthreads();
        // Y = Kb dS'   (Kb[i][k] = Kb^T[k][i])
        mmf<kChunk, kScanCols, kScanThreads>(
            kD, [&](int i, int k) { return col4(&s.KW[k * kP64 + i], kP64); },
            [&](int k, int j) { return col4(&s.D[k][j], kScanCols); },
            [&](int i, int j, float a) { s.Y[i][j] = a; });
        __syncthreads();
        put_w();
        __syncthreads();
        if (c > 0) fetch(c - 1);
        // dS = Diag(gamma) dS' - W^T Y + scale Q'^T dO
        mmf<kD, kScanCols, kScanThreads>(
            2 * kChunk,
            [&](int i, int k) {
                return k < kChunk ? scale4(col4(&s.KW[k * kP128 + i], kP128), -1.f)
                                  : scale4(col4(&s.QP[(k - kChunk) * kP128 + i], kP128), scale);
            },
            [&](int k, int j) {
                return k < kChunk ? col4(&s.Y[k][j], kScanCols) : col4(&s.O[k - kChunk][j], kScanCols);
            },
            [&](int i, int j, float a) { s.D[i][j] = fmaf(s.gam[i], s.D[i][j], a); });
    }
    __syncthreads();
    if (dh0)
        for (int e = tid; e < kD * kScanCols; e += kScanThreads) {
            const int i = e / kScanCols, j = e % kScanCols;
            dh0[(size_t)bh * kStateFloats + (size_t)i * kD + col0 + j] = s.D[i][j];
        }
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
// LDS: three [64][132] arrays (kh, qh and Gam while P and N are formed, then
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
    float(*const A0)[kPB] = s.big[0];  // kh, Kt, R, then dR
    float(*const A1)[kPB] = s.big[1];  // qh, Kb, dU, then scale dO
    float(*const A2)[kPB] = s.big[2];  // Gam, then U
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

    // ---- loads: q, k, g (8 threads per row, 16 channels each), then X and the
    // column strips of S and dS' (B operands of R and dU), v and dout
    float scol[32], dcol[32];  // S, dS' at [16 kb + 4 gq + e][cc], slot 4 kb + e
    typename RW::one vraw[16], oraw[16];
    float4 xpf[2];
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
        const float* Xg = xs + (size_t)blockIdx.x * kChunk * kChunk;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = tid + kCT * j;
            xpf[j] = ld4(Xg + (e >> 4) * kChunk + 4 * (e & 15));
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
        // the tiles of P and N above the diagonal blocks are zero
        for (int idx = tid; idx < kChunk * kChunk; idx += kCT) {
            const int i = idx >> 6, j = idx & 63;
            if (j >= 16 * ((i >> 4) + 1)) {
                s.p[i][j] = 0.f;
                s.n[i][j] = 0.f;
            }
        }
    }
    __syncthreads();

    // ---- P (strict lower) and N (lower incl) on the matrix cores -------------
    // For column block cb (i in 16 cb .. 16 cb + 15, reference row e = 16 cb +
    // 15) and rows r >= 16 cb: exp(Gam_r - Gam_i) = exp(Gam_r - Gam_e) exp(Gam_e -
    // Gam_i), both factors within exp(+-75) for g >= -5, so
    //   P_ri = sum_c (kh_rc exp(Gam_rc - Gam_ec)) (kh_ic exp(Gam_ec - Gam_ic)),
    // N likewise with qh_r.
    for (int t = wv; t < 10; t += kCT / 64) {  // the 10 tiles (rt, cb), rt >= cb
        int cb = 0, rem = t;
        while (rem >= 4 - cb) {
            rem -= 4 - cb;
            ++cb;
        }
        const int rt = cb + rem;
        const int r = 16 * rt + n, i = 16 * cb + n, e = 16 * cb + 15;
        f32x4 accp = {0.f, 0.f, 0.f, 0.f}, accn = {0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < kD; k0 += 16) {
            const int col = k0 + 4 * gq;
            const float4 gr = ld4(&A2[r][col]), ge = ld4(&A2[e][col]), gi = ld4(&A2[i][col]);
            const float4 f = exp4(make_float4(gr.x - ge.x, gr.y - ge.y, gr.z - ge.z, gr.w - ge.w));
            const float4 hh = exp4(make_float4(ge.x - gi.x, ge.y - gi.y, ge.z - gi.z, ge.w - gi.w));
            const float4 bk = mul4(ld4(&A0[i][col]), hh);
            mfma4(accp, mul4(ld4(&A0[r][col]), f), bk);
            mfma4(accn, mul4(ld4(&A1[r][col]), f), bk);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = 16 * rt + 4 * gq + u, col = 16 * cb + n;
            s.p[row][col] = col < row ? accp[u] : 0.f;
            s.n[row][col] = col <= row ? accn[u] : 0.f;
        }
    }
    // the lane's own kh, qh and Gam, kept in registers to the end
    float gmo[16], kho[16], qho[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int r = orow(m);
        gmo[m] = A2[r][cc];
        kho[m] = A0[r][cc];
        qho[m] = A1[r][cc];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = tid + kCT * j;
        *reinterpret_cast<float4*>(&s.x[e >> 4][4 * (e & 15)]) = xpf[j];
    }
    __syncthreads();  // P and N are done with kh, qh and Gam
    // -Kt = -e^Gam kh over kh and Kb = e^(GL - Gam) kh over qh, in 16-byte pieces
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid + kCT * j, r = e >> 5, c4 = 4 * (e & 31);
        const float4 kh = ld4(&A0[r][c4]), gm = ld4(&A2[r][c4]), gl = ld4(&s.gl[c4]);
        const float4 et = exp4(gm);
        const float4 eb = exp4(make_float4(gl.x - gm.x, gl.y - gm.y, gl.z - gm.z, gl.w - gm.w));
        *reinterpret_cast<float4*>(&A0[r][c4]) = scale4(mul4(et, kh), -1.f);
        *reinterpret_cast<float4*>(&A1[r][c4]) = mul4(eb, kh);
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
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            const float4 bs = make_float4(scol[4 * kb], scol[4 * kb + 1], scol[4 * kb + 2],
                                          scol[4 * kb + 3]);
            const float4 bd = make_float4(dcol[4 * kb], dcol[4 * kb + 1], dcol[4 * kb + 2],
                                          dcol[4 * kb + 3]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                mfma4(aR[u], ld4(&A0[16 * u + n][16 * kb + 4 * gq]), bs);
                mfma4(aU[u], ld4(&A1[16 * u + n][16 * kb + 4 * gq]), bd);
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
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int r = orow(m);
            dRo[m] = s.beta[r] * aD[m >> 2][m & 3];
            if (r < L) io_st(dv + base + (size_t)r * rp + cc, dRo[m]);
            A0[r][cc] = Ro[m];
            A1[r][cc] = dUo[m];
            A2[r][cc] = aX[m >> 2][m & 3];
        }
    }
    __syncthreads();  // R, dU and U are in LDS

    // ---- the 64 x 64 products: wave w computes tiles (rt0, ct) and (rt0 + 2, ct)
    const int ct = wv & 3, rt0 = wv >> 2;
    // dT = lower-incl(dU R^T); dbeta_j = sum_i X_ij dT_ij; dX = dT diag(beta)
    float dXo[8];
    {
        f32x4 aT[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            const float4 bR = ld4(&A0[16 * ct + n][16 * kb + 4 * gq]);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                if (rt0 + 2 * t >= ct) mfma4(aT[t], ld4(&A1[16 * (rt0 + 2 * t) + n][16 * kb + 4 * gq]), bR);
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
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int r = orow(m);
        A1[r][cc] = r < L ? scale * RW::wid(oraw[m]) : 0.f;
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
        for (int kb = 0; kb < 8; ++kb) {
            const float4 bU = ld4(&A2[16 * ct + n][16 * kb + 4 * gq]);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                if (rt0 + 2 * t >= ct) mfma4(aM[t], ld4(&A1[16 * (rt0 + 2 * t) + n][16 * kb + 4 * gq]), bU);
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
#pragma unroll
    for (int m = 0; m < 16; ++m) A0[orow(m)][cc] = dRo[m];
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
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                mfma4(aQ[u], ld4(&A1[16 * u + n][16 * kb + 4 * gq]), srow[kb]);
                mfma4(aK[u], ld4(&A0[16 * u + n][16 * kb + 4 * gq]), srow[kb]);
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
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int u = 0; u < 4; ++u) mfma4(aB[u], ld4(&A2[16 * u + n][16 * kb + 4 * gq]), drow[kb]);
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
           (RF::BYTES + (2 * kStateFloats + (size_t)kChunk * kChunk) * sizeof(float));
}

namespace {
// Workspace of a segment of nch chunks: records, then the states entering the
// chunks, the state gradients leaving them and X.
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
                                  hipStream_t stream) {
    const SegWs w(ws, B, H, nch);
    hipError_t e = launch_chunk_prep_f32(q, k, g, beta, B, T, H, chunk0, nch, w.rec, stream);
    if (e != hipSuccess) return e;
    const unsigned nscan = (unsigned)((int64_t)B * H * kScanSlices);
    hipLaunchKernelGGL(kda_bwd_state_scan_kernel<IO>, dim3(nscan), dim3(kScanThreads), 0, stream,
                       w.rec, v, h_in, w.states, h_out, T, H, chunk0, nch);
    return hipGetLastError();
}

template <typename IO>
hipError_t launch_chunk_bwd_segment(const IO* q, const IO* k, const IO* v, const float* g,
                                    const float* beta, float scale, const float* h_in,
                                    const IO* dout, const float* dS_in, IO* dq, IO* dk, IO* dv,
                                    float* dg, float* dbeta, float* dS_out, int B, int T, int H,
                                    int chunk0, int nch, void* ws, hipStream_t stream) {
    const SegWs w(ws, B, H, nch);
    hipError_t e =
        launch_chunk_prep_f32(q, k, g, beta, B, T, H, chunk0, nch, w.rec, stream, w.xs);
    if (e != hipSuccess) return e;
    const unsigned nscan = (unsigned)((int64_t)B * H * kScanSlices);
    hipLaunchKernelGGL(kda_bwd_state_scan_kernel<IO>, dim3(nscan), dim3(kScanThreads), 0, stream,
                       w.rec, v, h_in, w.states, nullptr, T, H, chunk0, nch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(kda_bwd_grad_scan_kernel<IO>, dim3(nscan), dim3(kScanThreads), 0, stream,
                       w.rec, dout, dS_in, w.dsn, dS_out, scale, T, H, chunk0, nch);
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
                                                   hipStream_t);                                 \
    template hipError_t launch_chunk_bwd_segment<IO>(                                            \
        const IO*, const IO*, const IO*, const float*, const float*, float, const float*,        \
        const IO*, const float*, IO*, IO*, IO*, float*, float*, float*, int, int, int, int, int, \
        void*, hipStream_t);
KDA_INST_BWD(float)
KDA_INST_BWD(uint16_t)
#undef KDA_INST_BWD

}  // namespace kda
