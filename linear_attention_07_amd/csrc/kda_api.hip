// The libkda C-ABI: argument validation, segmentation of long sequences,
// workspace from a library-owned stream-ordered pool, and kernel launches.
// Every KDA_ERR_INVALID_ARG / KDA_ERR_UNSUPPORTED decision is taken before the
// first HIP call, so it can be exercised on a machine without a GPU.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_common.hpp"
#include "kda_debug.hpp"
#include "kda_launch.hpp"

namespace {

constexpr int64_t kMaxBlocks = (int64_t)1 << 23;  // keeps blocks * threads < 2^32

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// Workspace budget for one segment of the chunked paths: default_mb (4 GB for
// the prefill, a 64K-token 96-head layer in one segment; 8 GB for the
// backward, an 8K-token 96-head layer in one segment); longer sequences are
// split.  The environment variable KDA_WORKSPACE_MB overrides both; it is read
// on every call, so a caller can force small segments.
size_t workspace_budget(size_t default_mb = 4096) {
    size_t mb = default_mb;
    if (const char* s = getenv("KDA_WORKSPACE_MB")) {
        const long v = strtol(s, nullptr, 10);
        if (v > 0) mb = (size_t)v;
    }
    return mb << 20;
}

long env_long(const char* name, long dflt) {
    const char* s = getenv(name);
    if (!s || !*s) return dflt;
    char* end = nullptr;
    const long v = strtol(s, &end, 10);
    return end && *end == '\0' ? v : dflt;
}

// One memory pool per device, created on first use, that keeps freed blocks
// cached so repeated calls do not go back to the driver (kda_trim_workspace
// hands them back).  Plain arrays and a mutex with trivial destructors: nothing
// here runs at process exit.
constexpr int kMaxDevices = 64;
std::mutex g_pool_mu;
hipMemPool_t g_pools[kMaxDevices] = {};

hipError_t pool_for_device(hipMemPool_t* pool) {
    std::mutex& mu = g_pool_mu;
    hipMemPool_t* pools = g_pools;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!pools[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t p = nullptr;
        e = hipMemPoolCreate(&p, &props);
        if (e != hipSuccess) return e;
        uint64_t keep = UINT64_MAX;
        e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep);
        if (e != hipSuccess) return e;
        pools[dev] = p;
    }
    *pool = pools[dev];
    return hipSuccess;
}

// The workspace of kda_chunk_fwd_noalloc: a device array of fixed size per GPU
// instead of the pool.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

// The scratch of kda_chunk_fwd_noalloc: 64 MiB per GPU, part of the library's
// code object, so each device that runs the library holds its own copy from
// the first use until the process ends.  Host code never uses its name as an
// address: the device address comes from hipGetSymbolAddress, once per device.
__device__ __align__(256) uint8_t kda_noalloc_scratch[kNoAllocScratchBytes];

namespace {

// the current device's copy of the scratch (device address)
hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(kda_noalloc_scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

// F32: fp32 q / k / v / out (else bf16); G16: bf16 g (else fp32; bf16 I/O only).
// conv.wq != NULL: q, k, v are raw values before the short convolution (bf16
// I/O only); conv_out (or NULL) receives the conv state after the sequence.
// no_alloc: the records and the carried state live in the fixed per-GPU
// scratch array (segments as long as it allows) and nothing is allocated.
template <bool F32, bool G16 = false>
kda_status_t chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                       const float* beta, float scale, const float* h0, void* out, float* hT,
                       int B, int T, int H, hipStream_t stream, kda::ConvArgs conv = {},
                       void* conv_out = nullptr, bool no_alloc = false) {
    static_assert(!(F32 && G16), "bf16 g is offered with bf16 q / k / v only");
    const bool cv = conv.wq != nullptr;
    constexpr size_t es = F32 ? 4 : 2;
    constexpr size_t gs = G16 ? 2 : 4;
    if (B < 0 || T < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    if (B == 0 || H == 0) return KDA_OK;
    const size_t state_bytes = (size_t)B * H * KDA_HEAD_DIM * KDA_HEAD_DIM * sizeof(float);
    if ((h0 && !aligned(h0, 16)) || (hT && !aligned(hT, 16))) return KDA_ERR_INVALID_ARG;
    if (h0 && hT && h0 != hT && overlap(h0, state_bytes, hT, state_bytes))
        return KDA_ERR_INVALID_ARG;
    if ((int64_t)B * H > kMaxBlocks) return KDA_ERR_UNSUPPORTED;
    // the short convolution's taps and state buffers
    const size_t wbytes = (size_t)H * KDA_HEAD_DIM * 4 * sizeof(float);
    const size_t cbytes = (size_t)3 * B * 3 * H * KDA_HEAD_DIM * sizeof(uint16_t);
    if (cv) {
        if (!conv.wk || !conv.wv) return KDA_ERR_INVALID_ARG;
        if (!aligned(conv.wq, 16) || !aligned(conv.wk, 16) || !aligned(conv.wv, 16) ||
            (conv.state && !aligned(conv.state, 16)) || (conv_out && !aligned(conv_out, 16)))
            return KDA_ERR_INVALID_ARG;
        if (conv.state && conv_out && conv.state != conv_out &&
            overlap(conv.state, cbytes, conv_out, cbytes))
            return KDA_ERR_INVALID_ARG;
        conv.B = B;
    }

    if (T == 0) {
        if (cv && conv_out && conv_out != conv.state) {
            // no tokens: the state passes through (zeros if there is none)
            const hipError_t e = kda::launch_conv_state_out(nullptr, nullptr, nullptr, B, 0, H,
                                                            conv, conv_out, stream);
            if (e != hipSuccess) return KDA_ERR_HIP;
        }
        if (!hT || hT == h0) return KDA_OK;
        const hipError_t e =
            kda::launch_copy_or_zero(h0, hT, state_bytes / sizeof(float), stream);
        return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    if (!q || !k || !v || !g || !beta || !out) return KDA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 16) ||
        !aligned(out, 16) || !aligned(beta, 4))
        return KDA_ERR_INVALID_ARG;
    const size_t n_tok = (size_t)B * T * H;
    const size_t io_bytes = n_tok * KDA_HEAD_DIM * es;
    const void* ins[] = {q, k, v};
    for (const void* p : ins)
        if (overlap(out, io_bytes, p, io_bytes)) return KDA_ERR_INVALID_ARG;
    if (overlap(out, io_bytes, g, n_tok * KDA_HEAD_DIM * gs) ||
        overlap(out, io_bytes, beta, n_tok * 4) || overlap(out, io_bytes, h0, state_bytes) ||
        overlap(out, io_bytes, hT, state_bytes))
        return KDA_ERR_INVALID_ARG;
    if (cv) {
        const void* ws_[] = {conv.wq, conv.wk, conv.wv};
        for (const void* p : ws_)
            if (overlap(out, io_bytes, p, wbytes) || overlap(conv_out, cbytes, p, wbytes))
                return KDA_ERR_INVALID_ARG;
        if (overlap(out, io_bytes, conv.state, cbytes) || overlap(out, io_bytes, conv_out, cbytes))
            return KDA_ERR_INVALID_ARG;
        if (conv.gate && (!aligned(conv.gate, 16) || overlap(out, io_bytes, conv.gate, io_bytes) ||
                          overlap(conv_out, cbytes, conv.gate, io_bytes)))
            return KDA_ERR_INVALID_ARG;
        for (const void* p : ins)
            if (overlap(conv_out, cbytes, p, io_bytes)) return KDA_ERR_INVALID_ARG;
    }

    const int slices = F32 ? kda::chunk_f32_slices() : kda::chunk16_slices();
    if ((int64_t)B * H * slices > kMaxBlocks) return KDA_ERR_UNSUPPORTED;
    constexpr bool v16 = !F32;  // bf16: prep16 / scan16; fp32 I/O: the fp32 kernels
    const int nch = (T + 63) / 64;
    const size_t rec = v16 ? kda::chunk16_record_bytes() : kda::chunk_f32_record_bytes();
    const size_t per_chunk = (size_t)B * H * rec;
    int seg;
    if (!no_alloc) {
        seg = (int)(workspace_budget() / per_chunk);
        if (seg < 1) seg = 1;
    } else if (per_chunk * (size_t)nch <= kNoAllocScratchBytes) {
        seg = nch;  // one segment, no carried state
    } else {
        // records of seg chunks, then the state carried between segments
        seg = kNoAllocScratchBytes < state_bytes
                  ? 0
                  : (int)((kNoAllocScratchBytes - state_bytes) / per_chunk);
        if (seg < 1) return KDA_ERR_UNSUPPORTED;  // B * H too large for the scratch
    }
    if (seg > nch) seg = nch;
    if ((int64_t)B * H * seg > kMaxBlocks) seg = (int)(kMaxBlocks / ((int64_t)B * H));
    if (seg < 1) return KDA_ERR_UNSUPPORTED;
    const bool multi = seg < nch;

    kda::DebugScope dbg(stream);
    if (dbg.on()) {
        if (dbg.setup_status() != KDA_OK) return dbg.setup_status();
        const size_t nel = n_tok * KDA_HEAD_DIM;
        if constexpr (F32) {
            dbg.finite(static_cast<const float*>(q), nel);
            dbg.finite(static_cast<const float*>(k), nel);
            dbg.finite(static_cast<const float*>(v), nel);
        } else {
            dbg.finite(static_cast<const uint16_t*>(q), nel);
            dbg.finite(static_cast<const uint16_t*>(k), nel);
            dbg.finite(static_cast<const uint16_t*>(v), nel);
        }
        if constexpr (G16)
            dbg.decay(static_cast<const uint16_t*>(g), nel);
        else
            dbg.decay(static_cast<const float*>(g), nel);
        dbg.finite(beta, n_tok);
        dbg.finite(h0, state_bytes / sizeof(float));
        if (cv) {
            const size_t nw = wbytes / sizeof(float);
            dbg.finite(conv.wq, nw);
            dbg.finite(conv.wk, nw);
            dbg.finite(conv.wv, nw);
            dbg.finite(conv.state, cbytes / sizeof(uint16_t));
            dbg.finite(conv.gate, nel);
        }
        const kda_status_t st = dbg.inputs_status();
        if (st != KDA_OK) return st;
    }
    kda::WaitCtl wait;
    wait.abort_out = dbg.abort_word();
    wait.spin_limit = dbg.spin_limit();

    void* ws = nullptr;
    float* carry = nullptr;
    if (no_alloc) {
        if (noalloc_scratch(&ws) != hipSuccess) return KDA_ERR_HIP;
        if (multi) carry = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + per_chunk * seg);
    } else {
        hipMemPool_t pool = nullptr;
        if (pool_for_device(&pool) != hipSuccess) return KDA_ERR_HIP;
        if (hipMallocFromPoolAsync(&ws, per_chunk * seg, pool, stream) != hipSuccess)
            return KDA_ERR_NO_MEMORY;
        if (multi) {
            if (hipMallocFromPoolAsync((void**)&carry, state_bytes, pool, stream) != hipSuccess) {
                (void)hipFreeAsync(ws, stream);
                return KDA_ERR_NO_MEMORY;
            }
        }
    }

    kda_status_t st = KDA_OK;
    for (int c0 = 0; c0 < nch; c0 += seg) {
        const int n = (nch - c0 < seg) ? nch - c0 : seg;
        const bool last = c0 + n >= nch;
        const float* h_in = (c0 == 0) ? h0 : carry;
        float* h_out = last ? (hT ? hT : nullptr) : carry;
        hipError_t e1, e2;
        if constexpr (v16) {
            e1 = kda::launch_prep16(q, k, g, G16, beta, B, T, H, c0, n, ws, conv, stream);
            e2 = e1 == hipSuccess ? kda::launch_scan16(ws, v, h_in, h_out, out, scale, B, T, H, c0,
                                                       n, conv, wait, stream)
                                  : e1;
        } else {
            e1 = kda::launch_chunk_prep_f32(static_cast<const float*>(q),
                                            static_cast<const float*>(k),
                                            static_cast<const float*>(g), beta, B, T, H, c0, n,
                                            ws, stream);
            e2 = e1 == hipSuccess
                     ? kda::launch_chunk_scan_f32(ws, static_cast<const float*>(v), h_in, h_out,
                                                  static_cast<float*>(out), scale, B, T, H, c0, n,
                                                  wait, stream)
                     : e1;
        }
        if (e2 != hipSuccess) {
            st = KDA_ERR_HIP;
            break;
        }
    }
    // the conv state after the sequence, once every segment has read the one
    // before it (conv_out may be the same buffer)
    if (st == KDA_OK && cv && conv_out &&
        kda::launch_conv_state_out(q, k, v, B, T, H, conv, conv_out, stream) != hipSuccess)
        st = KDA_ERR_HIP;
    if (!no_alloc) {
        if (carry) (void)hipFreeAsync(carry, stream);
        (void)hipFreeAsync(ws, stream);
    }
    if (st == KDA_OK && dbg.on()) st = dbg.device_status();
    return st;
}

// Backward of the chunked prefill; see kda_chunk_bwd_f32 and kda_chunk_bwd in
// kda.h.  IO: float, or uint16_t for bf16 q / k / v / dout / dq / dk / dv.
template <typename IO>
kda_status_t chunk_bwd(const IO* q, const IO* k, const IO* v, const float* g, const float* beta,
                       float scale, const float* h0, const IO* dout, const float* dhT, IO* dq,
                       IO* dk, IO* dv, float* dg, float* dbeta, float* dh0, int B, int T, int H,
                       hipStream_t stream) {
    if (B < 0 || T < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    if (B == 0 || H == 0) return KDA_OK;
    const size_t sbytes = (size_t)B * H * KDA_HEAD_DIM * KDA_HEAD_DIM * sizeof(float);
    const float* states[] = {h0, dhT, dh0};
    for (const float* p : states)
        if (p && !aligned(p, 16)) return KDA_ERR_INVALID_ARG;
    if (dh0 && (overlap(dh0, sbytes, h0, sbytes) || overlap(dh0, sbytes, dhT, sbytes)))
        return KDA_ERR_INVALID_ARG;
    if ((int64_t)B * H > kMaxBlocks) return KDA_ERR_UNSUPPORTED;
    if (T == 0) {  // no tokens: the state gradient passes through
        if (!dh0) return KDA_OK;
        const hipError_t e = kda::launch_copy_or_zero(dhT, dh0, sbytes / sizeof(float), stream);
        return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    const void* ptrs[] = {q, k, v, g, dout, dq, dk, dv, dg};
    for (const void* p : ptrs)
        if (!p || !aligned(p, 16)) return KDA_ERR_INVALID_ARG;
    if (!beta || !dbeta || !aligned(beta, 4) || !aligned(dbeta, 4)) return KDA_ERR_INVALID_ARG;
    const size_t n_tok = (size_t)B * T * H;
    // IO arrays (q, k, v, dout, dq, dk, dv) and fp32 ones (g, dg)
    const size_t vb = n_tok * KDA_HEAD_DIM * sizeof(IO), fb = n_tok * KDA_HEAD_DIM * sizeof(float);
    const size_t bb = n_tok * sizeof(float);
    // every written buffer overlaps no other argument
    struct Buf {
        const void* p;
        size_t n;
    };
    // argument slots; the written ones come last.  Two different slots may
    // never overlap when either is written, even at the same address.
    const Buf all[] = {{q, vb},  {k, vb},  {v, vb},      {g, fb},     {dout, vb},
                       {beta, bb}, {h0, sbytes}, {dhT, sbytes}, {dq, vb}, {dk, vb},
                       {dv, vb}, {dg, fb}, {dbeta, bb}, {dh0, sbytes}};
    constexpr int kSlots = sizeof(all) / sizeof(all[0]), kFirstWritten = 8;
    for (int w = kFirstWritten; w < kSlots; ++w)
        for (int a = 0; a < kSlots; ++a)
            if (a != w && overlap(all[w].p, all[w].n, all[a].p, all[a].n))
                return KDA_ERR_INVALID_ARG;
    if ((int64_t)B * H * 2 > kMaxBlocks) return KDA_ERR_UNSUPPORTED;  // two scan slices a head

    // Segments of seg chunks within the workspace budget (8 GB by default).
    // Segment s needs the state entering it: a forward pass over the segments
    // before the last keeps those states (checkpoints, one per segment), then
    // the segments are differentiated last to first, each recomputing its
    // records and states from its checkpoint, the state gradient carried from
    // one to the one before.  One segment (the whole sequence) needs neither.
    const int nch = (T + 63) / 64;
    const size_t per_chunk = kda::chunk_bwd_segment_bytes_per_chunk(B, H);
    int seg = (int)(workspace_budget(8192) / per_chunk);
    if (seg < 1) seg = 1;
    if (seg > nch) seg = nch;
    if ((int64_t)B * H * seg > kMaxBlocks) seg = (int)(kMaxBlocks / ((int64_t)B * H));
    if (seg < 1) return KDA_ERR_UNSUPPORTED;
    const int nseg = (nch + seg - 1) / seg;
    const size_t sfloats = sbytes / sizeof(float);

    kda::DebugScope dbg(stream);
    if (dbg.on()) {
        if (dbg.setup_status() != KDA_OK) return dbg.setup_status();
        const size_t nel = n_tok * KDA_HEAD_DIM;
        dbg.finite(q, nel);
        dbg.finite(k, nel);
        dbg.finite(v, nel);
        dbg.decay(g, nel);
        dbg.finite(beta, n_tok);
        dbg.finite(dout, nel);
        dbg.finite(h0, sfloats);
        dbg.finite(dhT, sfloats);
        const kda_status_t st = dbg.inputs_status();
        if (st != KDA_OK) return st;
    }

    hipMemPool_t pool = nullptr;
    if (pool_for_device(&pool) != hipSuccess) return KDA_ERR_HIP;
    // the segment's workspace, then the checkpoints of segments 1 .. nseg - 1
    // and the carried state gradient
    const size_t seg_bytes = per_chunk * seg;
    const size_t extra = nseg > 1 ? (size_t)nseg * sbytes : 0;
    void* ws = nullptr;
    if (hipMallocFromPoolAsync(&ws, seg_bytes + extra, pool, stream) != hipSuccess)
        return KDA_ERR_NO_MEMORY;
    float* ckpt = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + seg_bytes);
    kda::WaitCtl wait;
    wait.abort_out = dbg.abort_word();
    wait.spin_limit = dbg.spin_limit();
    float* dcarry = ckpt + (size_t)(nseg - 1) * sfloats;
    hipError_t e = hipSuccess;
    for (int sg = 0; sg + 1 < nseg && e == hipSuccess; ++sg)
        e = kda::launch_chunk_fwd_state<IO>(q, k, v, g, beta,
                                            sg == 0 ? h0 : ckpt + (size_t)(sg - 1) * sfloats,
                                            ckpt + (size_t)sg * sfloats, B, T, H, sg * seg, seg,
                                            ws, wait, stream);
    for (int sg = nseg - 1; sg >= 0 && e == hipSuccess; --sg) {
        const int c0 = sg * seg, n = nch - c0 < seg ? nch - c0 : seg;
        e = kda::launch_chunk_bwd_segment<IO>(
            q, k, v, g, beta, scale, sg == 0 ? h0 : ckpt + (size_t)(sg - 1) * sfloats, dout,
            sg == nseg - 1 ? dhT : dcarry, dq, dk, dv, dg, dbeta, sg == 0 ? dh0 : dcarry, B, T, H,
            c0, n, ws, wait, stream);
    }
    (void)hipFreeAsync(ws, stream);
    if (e != hipSuccess) return KDA_ERR_HIP;
    return dbg.on() ? dbg.device_status() : KDA_OK;
}

// conv != NULL: q, k, v are raw values before the short convolution (bf16 I/O
// only), and conv->state is advanced by one token in place.
template <bool F32>
kda_status_t recurrent_step(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, float scale, float* S, void* out, int B, int H,
                            hipStream_t stream, kda::DecodeConv* conv = nullptr) {
    constexpr size_t es = F32 ? 4 : 2;
    if (B < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    if (B == 0 || H == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !S || !out) return KDA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 16) ||
        !aligned(S, 16) || !aligned(out, 16) || !aligned(beta, 4))
        return KDA_ERR_INVALID_ARG;
    if ((int64_t)B * H > kMaxBlocks) return KDA_ERR_UNSUPPORTED;
    const size_t nbh = (size_t)B * H;
    const size_t vec = nbh * KDA_HEAD_DIM * es;
    const size_t sbytes = nbh * KDA_HEAD_DIM * KDA_HEAD_DIM * sizeof(float);
    const void* ins[] = {q, k, v};
    for (const void* p : ins)
        if (overlap(out, vec, p, vec) || overlap(S, sbytes, p, vec)) return KDA_ERR_INVALID_ARG;
    if (overlap(out, vec, g, nbh * KDA_HEAD_DIM * 4) || overlap(out, vec, beta, nbh * 4) ||
        overlap(out, vec, S, sbytes) || overlap(S, sbytes, g, nbh * KDA_HEAD_DIM * 4) ||
        overlap(S, sbytes, beta, nbh * 4))
        return KDA_ERR_INVALID_ARG;
    if (conv) {
        if (F32 || !conv->wq || !conv->wk || !conv->wv || !conv->state) return KDA_ERR_INVALID_ARG;
        if (!aligned(conv->wq, 16) || !aligned(conv->wk, 16) || !aligned(conv->wv, 16) ||
            !aligned(conv->state, 16))
            return KDA_ERR_INVALID_ARG;
        // the state is written: it may overlap nothing else
        const size_t cbytes = (size_t)3 * B * 3 * H * KDA_HEAD_DIM * sizeof(uint16_t);
        const size_t wbytes = (size_t)H * KDA_HEAD_DIM * 4 * sizeof(float);
        uint16_t* cs = conv->state;
        for (const void* p : ins)
            if (overlap(cs, cbytes, p, vec)) return KDA_ERR_INVALID_ARG;
        const void* taps[] = {conv->wq, conv->wk, conv->wv};
        for (const void* p : taps)
            if (overlap(cs, cbytes, p, wbytes) || overlap(out, vec, p, wbytes) ||
                overlap(S, sbytes, p, wbytes))
                return KDA_ERR_INVALID_ARG;
        if (overlap(cs, cbytes, g, nbh * KDA_HEAD_DIM * 4) || overlap(cs, cbytes, beta, nbh * 4) ||
            overlap(cs, cbytes, S, sbytes) || overlap(cs, cbytes, out, vec))
            return KDA_ERR_INVALID_ARG;
        if (conv->gate && (!aligned(conv->gate, 16) || overlap(out, vec, conv->gate, vec) ||
                           overlap(cs, cbytes, conv->gate, vec) ||
                           overlap(S, sbytes, conv->gate, vec)))
            return KDA_ERR_INVALID_ARG;
        conv->B = B;
        conv->H = H;
    }
    kda::DebugScope dbg(stream);
    if (dbg.on()) {
        if (dbg.setup_status() != KDA_OK) return dbg.setup_status();
        const size_t nel = nbh * KDA_HEAD_DIM;
        if constexpr (F32) {
            dbg.finite(static_cast<const float*>(q), nel);
            dbg.finite(static_cast<const float*>(k), nel);
            dbg.finite(static_cast<const float*>(v), nel);
        } else {
            dbg.finite(static_cast<const uint16_t*>(q), nel);
            dbg.finite(static_cast<const uint16_t*>(k), nel);
            dbg.finite(static_cast<const uint16_t*>(v), nel);
        }
        dbg.decay(g, nel);
        dbg.finite(beta, nbh);
        dbg.finite(S, nbh * KDA_HEAD_DIM * KDA_HEAD_DIM);
        if (conv) {
            const size_t nw = (size_t)H * KDA_HEAD_DIM * 4;
            dbg.finite(conv->wq, nw);
            dbg.finite(conv->wk, nw);
            dbg.finite(conv->wv, nw);
            dbg.finite(static_cast<const uint16_t*>(conv->state), (size_t)9 * nbh * KDA_HEAD_DIM);
            dbg.finite(conv->gate, nel);
        }
        const kda_status_t st = dbg.inputs_status();
        if (st != KDA_OK) return st;
    }
    const hipError_t e =
        kda::launch_decode<F32>(q, k, v, g, beta, scale, S, out, B, H, conv, stream);
    if (e != hipSuccess) return KDA_ERR_HIP;
    return dbg.on() ? dbg.device_status() : KDA_OK;
}

}  // namespace

namespace kda {

// The status words of the KDA_DEBUG_CHECKS mode, one array per GPU (each device
// holds its own copy at its own address): [0] a value outside its range, [1]
// a value not finite, [2] a bounded device wait gave up.
__device__ __align__(256) unsigned kda_debug_words[4];

namespace {
std::mutex g_words_mu;
unsigned* g_words[kMaxDevices] = {};

// the current device's status words (device address), looked up once per device
hipError_t debug_words(unsigned** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_words_mu);
    if (!g_words[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(kda_debug_words));
        if (e != hipSuccess) return e;
        g_words[dev] = static_cast<unsigned*>(p);
    }
    *out = g_words[dev];
    return hipSuccess;
}

template <bool BF16>
__global__ void kda_check_kernel(const void* __restrict__ p, size_t n, float lo, float hi,
                                 unsigned* __restrict__ flags) {
    bool out_of_range = false, not_finite = false;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float x = BF16 ? bf2f(static_cast<const uint16_t*>(p)[i])
                             : static_cast<const float*>(p)[i];
        if (lo <= hi && !(x >= lo && x <= hi)) out_of_range = true;
        if (!isfinite(x)) not_finite = true;
    }
    if (out_of_range) flags[0] = 1u;
    if (not_finite) flags[1] = 1u;
}
}  // namespace

hipError_t launch_check(const void* p, size_t n, bool bf16, float lo, float hi,
                        unsigned* flags, hipStream_t stream) {
    if (!p || n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (bf16)
        hipLaunchKernelGGL(kda_check_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           p, n, lo, hi, flags);
    else
        hipLaunchKernelGGL(kda_check_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           p, n, lo, hi, flags);
    return hipGetLastError();
}

DebugScope::DebugScope(hipStream_t stream) : stream_(stream) {
    on_ = env_long("KDA_DEBUG_CHECKS", 0) != 0;
    if (!on_) return;
    const long lim = env_long("KDA_DEBUG_SPIN_LIMIT", 0);
    if (lim > 0) spin_ = (unsigned)(lim < (long)kDefaultSpinLimit ? lim : kDefaultSpinLimit);
    if (debug_words(&flags_) != hipSuccess ||
        launch_copy_or_zero(nullptr, reinterpret_cast<float*>(flags_), 4, stream_) != hipSuccess)
        setup_ = KDA_ERR_HIP;
}

void DebugScope::check(const void* p, size_t n, bool bf16, float lo, float hi) {
    if (!on_ || setup_ != KDA_OK || !p) return;
    if (launch_check(p, n, bf16, lo, hi, flags_, stream_) != hipSuccess) launch_failed_ = true;
}

kda_status_t DebugScope::inputs_status() {
    if (!on_) return KDA_OK;
    if (setup_ != KDA_OK || launch_failed_) return KDA_ERR_HIP;
    unsigned w[4] = {0u, 0u, 0u, 0u};
    if (hipMemcpyAsync(w, flags_, sizeof(w), hipMemcpyDeviceToHost, stream_) != hipSuccess ||
        hipStreamSynchronize(stream_) != hipSuccess)
        return KDA_ERR_HIP;
    return (w[0] | w[1]) ? KDA_ERR_PRECONDITION : KDA_OK;
}

kda_status_t DebugScope::device_status() {
    if (!on_) return KDA_OK;
    unsigned w[4] = {0u, 0u, 0u, 0u};
    if (hipMemcpyAsync(w, flags_, sizeof(w), hipMemcpyDeviceToHost, stream_) != hipSuccess ||
        hipStreamSynchronize(stream_) != hipSuccess)
        return KDA_ERR_HIP;
    return w[2] ? KDA_ERR_DEVICE : KDA_OK;
}

__global__ void copy_or_zero_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                    size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_copy_or_zero(const float* src, float* dst, size_t n, hipStream_t stream) {
    size_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src,
                       dst, n);
    return hipGetLastError();
}

}  // namespace kda

extern "C" {

kda_status_t kda_chunk_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const float* g, const float* beta, float scale, const float* h0,
                           uint16_t* out, float* hT, int B, int T, int H, hipStream_t stream) {
    return chunk_fwd<false>(q, k, v, g, beta, scale, h0, out, hT, B, T, H, stream);
}

kda_status_t kda_chunk_fwd_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const float* g, const float* beta, float scale,
                                   const float* h0, uint16_t* out, float* hT, int B, int T, int H,
                                   hipStream_t stream) {
    return chunk_fwd<false>(q, k, v, g, beta, scale, h0, out, hT, B, T, H, stream, {}, nullptr,
                            true);
}

kda_status_t kda_chunk_fwd_g16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               const uint16_t* g, const float* beta, float scale, const float* h0,
                               uint16_t* out, float* hT, int B, int T, int H, hipStream_t stream) {
    return chunk_fwd<false, true>(q, k, v, g, beta, scale, h0, out, hT, B, T, H, stream);
}

kda_status_t kda_chunk_fwd_conv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const float* wq, const float* wk, const float* wv,
                                const uint16_t* conv_in, uint16_t* conv_out, const float* g,
                                const float* beta, float scale, const float* h0,
                                const uint16_t* gate, uint16_t* out, float* hT, int B, int T,
                                int H, hipStream_t stream) {
    if (!wq || !wk || !wv) return KDA_ERR_INVALID_ARG;
    kda::ConvArgs conv;
    conv.wq = wq;
    conv.wk = wk;
    conv.wv = wv;
    conv.state = conv_in;
    conv.gate = gate;
    return chunk_fwd<false>(q, k, v, g, beta, scale, h0, out, hT, B, T, H, stream, conv,
                            conv_out);
}

kda_status_t kda_chunk_fwd_f32(const float* q, const float* k, const float* v, const float* g,
                               const float* beta, float scale, const float* h0, float* out,
                               float* hT, int B, int T, int H, hipStream_t stream) {
    return chunk_fwd<true>(q, k, v, g, beta, scale, h0, out, hT, B, T, H, stream);
}

kda_status_t kda_recurrent_step(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const float* g, const float* beta, float scale, float* S_inout,
                                uint16_t* out, int B, int H, hipStream_t stream) {
    return recurrent_step<false>(q, k, v, g, beta, scale, S_inout, out, B, H, stream);
}

kda_status_t kda_recurrent_step_conv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const float* wq, const float* wk, const float* wv,
                                     uint16_t* conv_state, const float* g, const float* beta,
                                     float scale, float* S_inout, const uint16_t* gate,
                                     uint16_t* out, int B, int H, hipStream_t stream) {
    kda::DecodeConv conv;
    conv.wq = wq;
    conv.wk = wk;
    conv.wv = wv;
    conv.state = conv_state;
    conv.gate = gate;
    return recurrent_step<false>(q, k, v, g, beta, scale, S_inout, out, B, H, stream, &conv);
}

kda_status_t kda_recurrent_step_f32(const float* q, const float* k, const float* v,
                                    const float* g, const float* beta, float scale,
                                    float* S_inout, float* out, int B, int H,
                                    hipStream_t stream) {
    return recurrent_step<true>(q, k, v, g, beta, scale, S_inout, out, B, H, stream);
}

kda_status_t kda_chunk_bwd_f32(const float* q, const float* k, const float* v, const float* g,
                               const float* beta, float scale, const float* h0,
                               const float* dout, const float* dhT, float* dq, float* dk,
                               float* dv, float* dg, float* dbeta, float* dh0, int B, int T,
                               int H, hipStream_t stream) {
    return chunk_bwd<float>(q, k, v, g, beta, scale, h0, dout, dhT, dq, dk, dv, dg, dbeta, dh0,
                            B, T, H, stream);
}

kda_status_t kda_chunk_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const float* g, const float* beta, float scale, const float* h0,
                           const uint16_t* dout, const float* dhT, uint16_t* dq, uint16_t* dk,
                           uint16_t* dv, float* dg, float* dbeta, float* dh0, int B, int T, int H,
                           hipStream_t stream) {
    return chunk_bwd<uint16_t>(q, k, v, g, beta, scale, h0, dout, dhT, dq, dk, dv, dg, dbeta,
                               dh0, B, T, H, stream);
}

kda_status_t kda_trim_workspace(void) {
    std::lock_guard<std::mutex> lock(g_pool_mu);
    for (int d = 0; d < kMaxDevices; ++d)
        if (g_pools[d] && hipMemPoolTrimTo(g_pools[d], 0) != hipSuccess) return KDA_ERR_HIP;
    return KDA_OK;
}

const char* kda_status_string(kda_status_t s) {
    switch (s) {
        case KDA_OK: return "KDA_OK: success";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: invalid argument";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: size not supported";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: HIP runtime or launch error";
        case KDA_ERR_NO_MEMORY: return "KDA_ERR_NO_MEMORY: workspace allocation failed";
        case KDA_ERR_PRECONDITION:
            return "KDA_ERR_PRECONDITION: an input breaks a precondition (g outside [-5, 0] or a "
                   "value not finite; KDA_DEBUG_CHECKS)";
        case KDA_ERR_DEVICE:
            return "KDA_ERR_DEVICE: a device wait gave up; the outputs are invalid "
                   "(KDA_DEBUG_CHECKS)";
    }
    return "KDA: unknown status";
}

}  // extern "C"
