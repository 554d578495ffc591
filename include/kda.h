/*
 * libkda: the Kimi Delta Attention (KDA) forward pass on AMD MI355X (gfx950).
 *
 * KDA is a gated delta-rule linear attention.  Per batch entry b and head h a
 * 128 x 128 fp32 state S (row = key channel, column = value channel) evolves
 * token by token:
 *
 *   qh = q_t / |q_t|,  kh = k_t / |k_t|          (L2 norm, eps 1e-6 under the
 *                                                 square root, done inside)
 *   S  = Diag(exp g_t) S                          (per-channel decay, g <= 0)
 *   S += beta_t kh (v_t - S^T kh)^T               (delta-rule write)
 *   o_t = scale S^T qh                            (read-out after the write)
 *
 * Sources: Kimi-K3 深度解析 (d7kj.com blog), section 三 "KDA 的关键改进" for the
 * decay-then-correct recurrence and section 三 "Triton 实现" for the
 * chunkwise prefill; 深入 Kimi-K3 (xitter thread), KDA paragraph, for the
 * in-kernel q/k L2 normalisation, the per-channel decay with a -5 lower bound
 * on its logarithm, 96 heads of dimension 128 and the context-independent
 * state; Kimi K3 架构全景 page, section 02, for the two operations' names
 * (chunk_kda for prefill, fused_recurrent_kda for decode).
 *
 * Conventions for every entry point
 *   - d_k = d_v = 128 (KDA_HEAD_DIM), fixed.
 *   - bf16 tensors are raw uint16_t bit patterns (round-to-nearest-even when
 *     produced here).
 *   - Every pointer is DEVICE memory owned by the caller.  The library never
 *     frees, retains or reallocates a caller pointer after it returns.
 *   - Work is enqueued on `stream` and the call returns without
 *     synchronising.  A device fault surfaces at the caller's next sync.
 *   - Offsets are 64-bit: B*T*H*128 may exceed 2^31.
 *   - Precondition: g lies in [-5, 0].  The chunked path relies on the lower
 *     bound to keep its factorised decay in range; it is the bound the pages
 *     give for the decay gate.  It is not checked by default (the check reads
 *     every g); see KDA_DEBUG_CHECKS below.
 *   - Arguments are validated before any HIP call, so every
 *     KDA_ERR_INVALID_ARG case is reported without touching a GPU.
 *   - No exceptions cross the ABI; nothing is printed; nothing aborts.
 *
 * Environment (read on every call)
 *   - KDA_WORKSPACE_MB: workspace budget per segment of the chunked paths
 *     (default 4096 for the prefill, 8192 for its backward).  Long sequences
 *     are split into segments of as many 64-token chunks as fit.
 *   - KDA_DEBUG_CHECKS=1: before launching, every entry point scans its
 *     inputs on the device (g within [-5, 0]; q, k, v, beta, states, output
 *     gradients, taps, conv states and gate logits finite), synchronises its
 *     stream and returns KDA_ERR_PRECONDITION if one fails; after its work it
 *     synchronises again and returns KDA_ERR_DEVICE if a bounded device wait
 *     gave up.  The mode synchronises: it is not for graph capture.
 *   - KDA_DEBUG_SPIN_LIMIT=n (only with KDA_DEBUG_CHECKS): the polls a bounded
 *     wait makes before it gives up, to exercise the KDA_ERR_DEVICE path.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_HEAD_DIM 128

#if defined(__GNUC__)
#define KDA_API __attribute__((visibility("default")))
#else
#define KDA_API
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative size, bad scale */
    KDA_ERR_UNSUPPORTED = 2, /* a size the library cannot index (e.g. T > 2^31-1) */
    KDA_ERR_HIP = 3,         /* a HIP runtime call or launch failed */
    KDA_ERR_NO_MEMORY = 4,   /* internal workspace could not be allocated */
    KDA_ERR_PRECONDITION = 5, /* KDA_DEBUG_CHECKS: g outside [-5, 0] or a value not finite;
                                 nothing was launched */
    KDA_ERR_DEVICE = 6       /* KDA_DEBUG_CHECKS: a bounded device wait gave up; the outputs
                                are invalid */
} kda_status_t;

/*
 * kda_chunk_fwd — chunkwise-parallel prefill (the pages' chunk_kda).
 *
 *   q, k, v : [B, T, H, 128] bf16, row-major (channel fastest).
 *   g       : [B, T, H, 128] fp32 log-decay per key channel, in [-5, 0].
 *   beta    : [B, T, H] fp32, one scalar per token and head.
 *   scale   : read-out scale (finite); multiplies o only, never the state.
 *   h0      : [B, H, 128, 128] fp32 initial state (row = key channel), or
 *             NULL for a zero state.
 *   out     : [B, T, H, 128] bf16 output o.  Must not alias any input.
 *   hT      : [B, H, 128, 128] fp32 final state, or NULL to skip it.  hT may
 *             equal h0 (in-place carry of the state).
 *
 * Any T >= 0 is valid: T need not be a multiple of the internal chunk of 64
 * tokens.  T == 0 writes hT = h0 (zeros if h0 is NULL).  B == 0 or H == 0 is
 * a no-op.  Pointers must be 16-byte aligned.  The result equals the
 * token-by-token recurrence above up to floating-point rounding: the chunk
 * form is an exact rearrangement (UT/WY representation of the in-chunk
 * triangular system, products on bf16 matrix cores with fp32 accumulation,
 * state kept in fp32).  Internal workspace is taken from a library-owned,
 * stream-ordered memory pool and is bounded by splitting T into segments.
 */
KDA_API kda_status_t kda_chunk_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const float *g, const float *beta, float scale,
                           const float *h0, uint16_t *out, float *hT,
                           int B, int T, int H, hipStream_t stream);

/*
 * kda_chunk_fwd_noalloc — kda_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture that must not add allocation
 * nodes, tight serving loops, harnesses that forbid hipMalloc).  Arguments,
 * layouts, validation and results are those of kda_chunk_fwd, and the results
 * are bitwise the same.  Nothing is allocated: the per-chunk records and the
 * state carried between segments live in a fixed 64 MiB device array of the
 * library, one per GPU, held from its first use until the process ends; T is
 * split into as many segments as that array needs (about 9 chunks of 64
 * tokens per segment at B * H = 96), so long sequences take more launches.
 * Returns KDA_ERR_UNSUPPORTED, before any HIP call, when B * H is too large
 * for one chunk and the carried state to fit (B * H > 500 or so).  Calls on
 * one GPU share that GPU's array, so calls that overlap in time on one GPU
 * (on different streams, or from several host threads) race and give wrong
 * results; calls on one stream are ordered and safe.  Not with
 * KDA_DEBUG_CHECKS under graph capture (the mode synchronises).
 */
KDA_API kda_status_t kda_chunk_fwd_noalloc(const uint16_t *q, const uint16_t *k,
                                   const uint16_t *v, const float *g, const float *beta,
                                   float scale, const float *h0, uint16_t *out, float *hT,
                                   int B, int T, int H, hipStream_t stream);

/*
 * kda_chunk_fwd_g16 — as kda_chunk_fwd, with the log-decay in bf16:
 *
 *   g       : [B, T, H, 128] bf16 log-decay per key channel, in [-5, 0].
 *
 * Every other argument, the layout, the validation and the result are those
 * of kda_chunk_fwd; the bf16 values of g are used exactly (widened to fp32).
 * The decay is an input of the operation (its gate, a full-rank projection
 * bounded below by -5 on the Kimi K3 架构全景 page, section 02, is computed
 * before it), and the fp32 g stream is a third of the prefill's compulsory
 * bytes: in bf16 a token-head moves 1,284 instead of 1,540 bytes.
 */
KDA_API kda_status_t kda_chunk_fwd_g16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const uint16_t *g, const float *beta, float scale,
                               const float *h0, uint16_t *out, float *hT,
                               int B, int T, int H, hipStream_t stream);

/*
 * kda_chunk_fwd_conv — kda_chunk_fwd with the short convolution and SiLU that
 * the KDA layer puts in front of the attention, and optionally its output
 * gate behind it (the KDA paragraph of the
 * 深入 Kimi-K3 thread; a 4-tap kernel in the config table of the Kimi K3
 * architecture page), fused into the kernels' loads.  Read as depthwise and
 * causal with no bias: for each of q, k and v,
 *
 *   x'[b,t,h,c] = silu( sum_{j=0..3} w[h,c,j] * x[b,t-3+j,h,c] ),
 *   silu(a) = a / (1 + exp(-a)),
 *
 * where the tokens before t = 0 come from conv_in (zeros when it is NULL).
 * x' is rounded to bf16 and is then the q, k or v of kda_chunk_fwd.
 *
 *   q, k, v  : [B, T, H, 128] bf16 RAW values (before the convolution).
 *   wq/wk/wv : [H, 128, 4] fp32 taps; tap 3 weights the current token, tap j
 *              the token 3 - j steps before it.  Required; 16-byte aligned.
 *   conv_in  : NULL (a fresh sequence) or [3][B][3][H][128] bf16: for q, k, v
 *              in that order, the 3 raw tokens before the first one, oldest
 *              first.
 *   conv_out : NULL, or the same layout: receives the last 3 raw tokens of
 *              each tensor (taken from conv_in where T < 3), for the next
 *              call.  May equal conv_in (updated in place); otherwise must
 *              not overlap it, the weights or the inputs.
 *
 *   gate     : NULL, or [B, T, H, 128] bf16 logits z of the output gate
 *              behind the attention: out = o * sigmoid(z), elementwise, then
 *              rounded to bf16.  The 深入 Kimi-K3 thread (KDA paragraph) says
 *              only that K3's KDA output gate is full-rank, and that its
 *              global layers gate their output with a sigmoid; read here as
 *              a sigmoid of one logit per output channel (the projection
 *              that makes z, and any norm, stay outside).  16-byte aligned;
 *              must not overlap out or conv_out.
 *
 * g, beta, scale, h0, out, hT and the validation are those of kda_chunk_fwd;
 * out must not overlap the weights or the conv buffers either.  T == 0 copies
 * conv_in (or zeros) to conv_out and h0 (or zeros) to hT.
 */
KDA_API kda_status_t kda_chunk_fwd_conv(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const float *wq, const float *wk, const float *wv,
                                const uint16_t *conv_in, uint16_t *conv_out,
                                const float *g, const float *beta, float scale,
                                const float *h0, const uint16_t *gate, uint16_t *out,
                                float *hT, int B, int T, int H, hipStream_t stream);

/*
 * kda_chunk_fwd_f32 — as kda_chunk_fwd, with fp32 q, k, v and out (the
 * fp32-input accuracy mode).  Prep works in fp32 throughout, the inverse
 * included; the scan's products take each fp32 factor as a bf16 hi + lo pair
 * (three products per pair, fp32 accumulation, about 1e-5 relative per
 * product) and carry the state in fp32.  Measured against an fp64 reference:
 * normalised max errors about 1.5e-5 on outputs and 2e-5 on the final state.
 */
KDA_API kda_status_t kda_chunk_fwd_f32(const float *q, const float *k, const float *v,
                               const float *g, const float *beta, float scale,
                               const float *h0, float *out, float *hT,
                               int B, int T, int H, hipStream_t stream);

/*
 * kda_recurrent_step — one decode token over a maintained state (the pages'
 * fused_recurrent_kda).  The state replaces a KV cache: its size does not
 * depend on how many tokens came before.
 *
 *   q, k, v : [B, H, 128] bf16.
 *   g       : [B, H, 128] fp32 in [-5, 0].
 *   beta    : [B, H] fp32.
 *   scale   : finite read-out scale.
 *   S_inout : [B, H, 128, 128] fp32 state, updated in place.
 *   out     : [B, H, 128] bf16.  Must not alias any input or the state.
 *
 * B == 0 or H == 0 is a no-op.  Pointers must be 16-byte aligned.
 */
KDA_API kda_status_t kda_recurrent_step(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const float *g, const float *beta, float scale,
                                float *S_inout, uint16_t *out,
                                int B, int H, hipStream_t stream);

/*
 * kda_recurrent_step_conv — kda_recurrent_step with the short convolution and
 * SiLU in front of the attention (the same filter as kda_chunk_fwd_conv, read
 * as depthwise, causal, 4 taps, no bias), for decoding after a
 * kda_chunk_fwd_conv prefill:
 *
 *   x'[b,h,c] = silu( w[h,c,3] * x[b,h,c] + sum_{j=0..2} w[h,c,j] * st_x[b,j,h,c] ),
 *
 * rounded to bf16, is the q, k or v of kda_recurrent_step.
 *
 *   q, k, v    : [B, H, 128] bf16 RAW values of the new token.
 *   wq/wk/wv   : [H, 128, 4] fp32 taps, as in kda_chunk_fwd_conv.  Required.
 *   conv_state : [3][B][3][H][128] bf16, the layout kda_chunk_fwd_conv's
 *                conv_out writes: for q, k, v, the 3 raw tokens before this
 *                one, oldest first.  Required.  Updated in place: on return
 *                it holds the last 3 raw tokens including this one.  Must not
 *                overlap any other argument.
 *
 *   gate       : NULL, or [B, H, 128] bf16 logits of the output gate, as in
 *                kda_chunk_fwd_conv: out = o * sigmoid(gate).
 *
 * g, beta, scale, S_inout, out and the validation are those of
 * kda_recurrent_step; out must not overlap the taps, the conv state or the
 * gate.
 */
KDA_API kda_status_t kda_recurrent_step_conv(const uint16_t *q, const uint16_t *k,
                                     const uint16_t *v, const float *wq, const float *wk,
                                     const float *wv, uint16_t *conv_state,
                                     const float *g, const float *beta, float scale,
                                     float *S_inout, const uint16_t *gate, uint16_t *out,
                                     int B, int H, hipStream_t stream);

/* kda_recurrent_step_f32 — as kda_recurrent_step with fp32 q, k, v, out. */
KDA_API kda_status_t kda_recurrent_step_f32(const float *q, const float *k, const float *v,
                                    const float *g, const float *beta, float scale,
                                    float *S_inout, float *out,
                                    int B, int H, hipStream_t stream);

/*
 * kda_recurrent_step_bwd_f32 — backward of one kda_recurrent_step_f32 step,
 * for training through the recurrence one token at a time in reverse
 * (backpropagation through time, with the states before each step kept by
 * the caller).  The pages say only that the log-decay bound serves training
 * speed (ai-pulse-lab summary of the technical report, KDA paragraph); the
 * gradients are those of the step's assignments, differentiated in reverse
 * order.  For L = <dout, o> + <dS_next, S_new> of the step
 * (o, S_new) = step(q, k, v, g, beta, scale, S_prev):
 *
 *   q, k, v, g : [B, H, 128] fp32, the step's inputs (q, k raw: the L2 norms
 *                are differentiated too); beta [B, H] fp32; scale finite.
 *   S_prev     : [B, H, 128, 128] fp32, the state before the step.
 *   dout       : [B, H, 128] fp32, dL/do.
 *   dS         : [B, H, 128, 128] fp32, in: dL/dS_new (zeros after the last
 *                token); out: dL/dS_prev, in place, ready for the step before.
 *   dq, dk, dv, dg : [B, H, 128] fp32 outputs; dbeta [B, H] fp32 output.
 *
 * Every written buffer must not overlap any other argument.  All pointers
 * 16-byte aligned (beta, dbeta 4).  B == 0 or H == 0 is a no-op.
 */
KDA_API kda_status_t kda_recurrent_step_bwd_f32(const float *q, const float *k, const float *v,
                                        const float *g, const float *beta, float scale,
                                        const float *S_prev, const float *dout, float *dS,
                                        float *dq, float *dk, float *dv, float *dg,
                                        float *dbeta, int B, int H, hipStream_t stream);

/*
 * kda_recurrent_step_bwd — kda_recurrent_step_bwd_f32 for the bf16 decode
 * step kda_recurrent_step: q, k, v and dout are [B, H, 128] bf16, and dq, dk,
 * dv are written as [B, H, 128] bf16 (rounded to nearest even from fp32).
 * g, beta, S_prev, dS, dg and dbeta, the validation and the in-place update
 * of dS are those of kda_recurrent_step_bwd_f32.
 */
KDA_API kda_status_t kda_recurrent_step_bwd(const uint16_t *q, const uint16_t *k,
                                    const uint16_t *v, const float *g, const float *beta,
                                    float scale, const float *S_prev, const uint16_t *dout,
                                    float *dS, uint16_t *dq, uint16_t *dk, uint16_t *dv,
                                    float *dg, float *dbeta, int B, int H, hipStream_t stream);

/*
 * kda_chunk_bwd_f32 — backward of the fp32 chunked prefill kda_chunk_fwd_f32.
 *
 * The pages give no backward (they name training speed as the reason for the
 * decay's lower bound: ai-pulse-lab summary of the technical report, KDA
 * paragraph); the gradients are those of the recurrence of kda_chunk_fwd
 * (Kimi-K3 深度解析 blog, section 三), computed through its chunk form: for
 * L = <dout, o> + <dhT, hT> with (o, hT) = forward(q, k, v, g, beta, scale, h0),
 *
 *   q, k, v, g : [B, T, H, 128] fp32, the forward's inputs (q, k raw: the L2
 *                norms are differentiated too); beta [B, T, H] fp32.
 *   h0         : [B, H, 128, 128] fp32 initial state, or NULL for zeros.
 *   dout       : [B, T, H, 128] fp32, dL/do.
 *   dhT        : [B, H, 128, 128] fp32, dL/dhT, or NULL for zeros.
 *   dq, dk, dv, dg : [B, T, H, 128] fp32 outputs; dbeta [B, T, H] fp32 output.
 *   dh0        : [B, H, 128, 128] fp32 output dL/dh0, or NULL (not stored).
 *
 * Every written buffer must not overlap any other argument.  All pointers
 * 16-byte aligned (beta, dbeta 4).  B == 0 or H == 0 is a no-op; T == 0
 * copies dhT (or zeros) to dh0.  Workspace comes from the library's
 * stream-ordered pool (KDA_ERR_NO_MEMORY if it cannot be had) and is bounded
 * by the budget, not by T: the chunk records, three 64 x 64 matrices, the
 * state entering and the state gradient leaving every chunk (about 305 KB per
 * 64 tokens and head) are held for one segment of chunks at a time.  With more
 * than one segment, a forward pass first keeps the state entering each
 * segment (64 KB per segment and head), and the segments are then
 * differentiated last to first, each recomputing its states from its
 * checkpoint.  Computed in fp32 (the two state scans' products as three bf16
 * products of hi / lo pairs each, about 1e-5 relative per product, accumulated
 * in fp32); g obeys the forward's bound (every entry in [-5, 0]), which the
 * chunk records that the two state scans read rely on.
 */
KDA_API kda_status_t kda_chunk_bwd_f32(const float *q, const float *k, const float *v,
                               const float *g, const float *beta, float scale,
                               const float *h0, const float *dout, const float *dhT,
                               float *dq, float *dk, float *dv, float *dg, float *dbeta,
                               float *dh0, int B, int T, int H, hipStream_t stream);

/*
 * kda_chunk_bwd — kda_chunk_bwd_f32 for bf16 q, k, v and dout (the inputs of
 * kda_chunk_fwd): q, k, v, dout are [B, T, H, 128] bf16, and dq, dk, dv are
 * written as [B, T, H, 128] bf16 (rounded to nearest even from fp32).  g,
 * beta, the states, dg, dbeta and dh0 are fp32; all arithmetic is fp32.  The
 * gradients are those of the recurrence on the given bf16 values, not of the
 * bf16 forward kernel's own roundings.  Validation, workspace and the T == 0
 * case are those of kda_chunk_bwd_f32.
 */
KDA_API kda_status_t kda_chunk_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const float *g, const float *beta, float scale, const float *h0,
                           const uint16_t *dout, const float *dhT, uint16_t *dq,
                           uint16_t *dk, uint16_t *dv, float *dg, float *dbeta, float *dh0,
                           int B, int T, int H, hipStream_t stream);

/*
 * kda_trim_workspace — hands back to the driver the device memory that the
 * library's workspace pools keep cached between calls (one pool per device;
 * a 64K-token prefill keeps about 4 GB, an 8K-token backward about 4 GB).
 * Call it when no work of this library is in flight (after synchronising the
 * streams it ran on); memory still in use is not touched.  Returns KDA_OK, or
 * KDA_ERR_HIP.  Not needed before exit.
 */
KDA_API kda_status_t kda_trim_workspace(void);

/* Static, NUL-terminated description of a status code (never NULL). */
KDA_API const char *kda_status_string(kda_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
