// Internal host-side launch interface between the C-ABI layer (kda_api.hip)
// and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// The decode step's short convolution (bf16 I/O only): taps [H][128][4] fp32
// (tap 3 = the current token) and the conv state [3 (q, k, v)][B][3][H][128]
// bf16 (the 3 previous raw tokens, oldest first), advanced in place.
struct DecodeConv {
    const float* wq = nullptr;
    const float* wk = nullptr;
    const float* wv = nullptr;
    uint16_t* state = nullptr;
    const uint16_t* gate = nullptr;  // [B, H, 128] bf16 logits of the output gate, or NULL
    int B = 0;
    int H = 0;
};

// conv == NULL: q, k, v enter the attention as given
template <bool F32>
hipError_t launch_decode(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float scale, float* S, void* out,
                         int B, int H, const DecodeConv* conv, hipStream_t stream);

// two-kernel chunked prefill for fp32 q/k/v/o, fp32 arithmetic throughout.
// prep writes one record (W, Q', Kb^T, T, MT, gamma) per (batch, head, chunk)
// of chunks [chunk0, chunk0 + nchunks) into ws, from q, k, g, beta; scan walks
// them in order, reading v, the records and h_in (NULL = zero state), and
// writes out and, if h_out is not NULL, the final state.  x_out (or NULL)
// receives three [64][64] fp32 matrices per chunk, in record order: X = (I +
// A)^-1 (zero above the diagonal), P = strict-lower(KK) and N = M =
// lower-incl(QK) (zero above their diagonal blocks); prep then forms no M T.
size_t chunk_f32_record_bytes();
int chunk_f32_slices();
// Byte offsets inside one fp32 record (64-token chunks, 128 channels).
struct ChunkRecF32 {
    static constexpr size_t W = 0;                          // [64][128] W = T Kt
    static constexpr size_t QP = W + 64 * 128 * 4;          // [64][128] Q' = Qt - M W
    static constexpr size_t KT = QP + 64 * 128 * 4;         // [128][64] Kb^T
    static constexpr size_t TH = KT + 128 * 64 * 4;         // [64][64]  T
    static constexpr size_t MH = TH + 64 * 64 * 4;          // [64][64]  M T
    static constexpr size_t G = MH + 64 * 64 * 4;           // [128] gamma
    static constexpr size_t BYTES = ((G + 128 * 4) + 255) / 256 * 256;
};
hipError_t launch_chunk_prep_f32(const float* q, const float* k, const float* g,
                                 const float* beta, int B, int T, int H, int chunk0, int nchunks,
                                 void* ws, hipStream_t stream, float* x_out = nullptr);
// the same records (fp32) from bf16 q and k
hipError_t launch_chunk_prep_f32(const uint16_t* q, const uint16_t* k, const float* g,
                                 const float* beta, int B, int T, int H, int chunk0, int nchunks,
                                 void* ws, hipStream_t stream, float* x_out = nullptr);


// The scans' bounded LDS waits: their spin limit, and where a wait that gives
// up records it (NULL: nowhere).
struct WaitCtl {
    unsigned* abort_out = nullptr;
    unsigned spin_limit = 1u << 23;
};

hipError_t launch_chunk_scan_f32(const void* ws, const float* v, const float* h_in, float* h_out,
                                 float* out, float scale, int B, int T, int H, int chunk0,
                                 int nchunks, const WaitCtl& wait, hipStream_t stream);

// Backward of the chunked prefill over one segment of chunks [chunk0, chunk0 +
// nch): prep records, a forward scan storing the state entering each chunk
// (from h_in, the state entering chunk0; NULL = zeros), a reverse scan storing
// the state gradient leaving each chunk (from dS_in, the gradient of the state
// leaving the segment; NULL = zeros) and writing that of the state entering it
// to dS_out (NULL = not stored; may equal dS_in), and one gradient workgroup
// per chunk.  ws holds chunk_bwd_segment_bytes_per_chunk(B, H) * nch bytes.
// launch_chunk_fwd_state runs only the first two launches, and writes the
// state leaving the segment to h_out (the checkpoints of a segmented call).
// IO = float or uint16_t (bf16 q, k, v, dout in and dq, dk, dv out; all
// arithmetic fp32).
size_t chunk_bwd_segment_bytes_per_chunk(int B, int H);
template <typename IO>
hipError_t launch_chunk_fwd_state(const IO* q, const IO* k, const IO* v, const float* g,
                                  const float* beta, const float* h_in, float* h_out, int B,
                                  int T, int H, int chunk0, int nch, void* ws,
                                  const WaitCtl& wait, hipStream_t stream);
template <typename IO>
hipError_t launch_chunk_bwd_segment(const IO* q, const IO* k, const IO* v, const float* g,
                                    const float* beta, float scale, const float* h_in,
                                    const IO* dout, const float* dS_in, IO* dq, IO* dk, IO* dv,
                                    float* dg, float* dbeta, float* dS_out, int B, int T, int H,
                                    int chunk0, int nch, void* ws, const WaitCtl& wait,
                                    hipStream_t stream);

// Short convolution in front of the attention: depthwise 4-tap causal filter
// per head and channel, then SiLU, on q, k and v.  wq == NULL: none.  state:
// the 3 raw tokens before the sequence, [3 (q, k, v)][B][3][H][128] bf16, or
// NULL for zeros.
struct ConvArgs {
    const float* wq = nullptr;  // [H][128][4] fp32, tap 3 = the current token
    const float* wk = nullptr;
    const float* wv = nullptr;
    const uint16_t* state = nullptr;
    // optional output gate behind the attention: out = o * sigmoid(gate),
    // gate [B, T, H, 128] bf16 logits, or NULL for none
    const uint16_t* gate = nullptr;
    int B = 0;
};

// two-kernel chunked prefill for bf16 q/k/v/o: prep writes one record per
// (batch, head, chunk) of chunks [chunk0, chunk0 + nchunks) into ws, from g in
// fp32 or (g_bf16) bf16; scan walks them in order (h_in NULL = zero state,
// h_out NULL = final state not stored).
size_t chunk16_record_bytes();
int chunk16_slices();
hipError_t launch_prep16(const void* q, const void* k, const void* g, bool g_bf16,
                         const float* beta, int B, int T, int H, int chunk0, int nchunks, void* ws,
                         const ConvArgs& conv, hipStream_t stream);
hipError_t launch_scan16(const void* ws, const void* v, const float* h_in, float* h_out,
                         void* out, float scale, int B, int T, int H, int chunk0, int nchunks,
                         const ConvArgs& conv, const WaitCtl& wait, hipStream_t stream);
// the conv state after the sequence: the last 3 raw tokens of q, k, v (from
// the inputs, or from conv.state where T < 3), [3][B][3][H][128]; safe in
// place (st_out == conv.state)
hipError_t launch_conv_state_out(const void* q, const void* k, const void* v, int B, int T,
                                 int H, const ConvArgs& conv, void* st_out, hipStream_t stream);

// dst[i] = src ? src[i] : 0 for i < n (fp32), as a kernel so that it can be
// captured in a graph.
hipError_t launch_copy_or_zero(const float* src, float* dst, size_t n, hipStream_t stream);

}  // namespace kda
