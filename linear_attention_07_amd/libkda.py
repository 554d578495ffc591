"""Thin Python binding of the libkda C-ABI (``include/kda.h``).

Argument marshalling only: shapes, dtypes, contiguity and device are checked,
outputs are allocated with torch (device memory), and ``data_ptr()`` plus the
current HIP stream are handed to the C entry points.  Every step of the KDA
computation runs in the library's kernels; there is no fallback of any kind:
if ``libkda.so`` is missing this module raises on import of the library.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so libkda binds to the HIP runtime torch already holds

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libkda.so")
HEAD_DIM = 128

KDA_OK = 0
KDA_ERR_INVALID_ARG = 1
KDA_ERR_UNSUPPORTED = 2
KDA_ERR_HIP = 3
KDA_ERR_NO_MEMORY = 4
KDA_ERR_PRECONDITION = 5
KDA_ERR_DEVICE = 6

EXPORTS = (
    "kda_chunk_bwd",
    "kda_chunk_bwd_f32",
    "kda_chunk_fwd",
    "kda_chunk_fwd_conv",
    "kda_chunk_fwd_f32",
    "kda_chunk_fwd_g16",
    "kda_chunk_fwd_noalloc",
    "kda_recurrent_step",
    "kda_recurrent_step_bwd",
    "kda_recurrent_step_bwd_f32",
    "kda_recurrent_step_conv",
    "kda_recurrent_step_f32",
    "kda_status_string",
    "kda_trim_workspace",
)

_lib = None


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def load() -> ctypes.CDLL:
    """Load libkda.so (built by ``linear_attention_07_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m linear_attention_07_amd.build`"
        )
    lib = ctypes.CDLL(LIB_PATH)
    vp, f, i = ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    chunk_args = [vp, vp, vp, vp, vp, f, vp, vp, vp, i, i, i, vp]
    step_args = [vp, vp, vp, vp, vp, f, vp, vp, i, i, vp]
    conv_args = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f, vp, vp, vp, vp, i, i, i, vp]
    for name, args in (("kda_chunk_fwd", chunk_args), ("kda_chunk_fwd_f32", chunk_args),
                       ("kda_chunk_fwd_g16", chunk_args), ("kda_chunk_fwd_noalloc", chunk_args),
                       ("kda_chunk_fwd_conv", conv_args),
                       ("kda_recurrent_step", step_args), ("kda_recurrent_step_f32", step_args)):
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.kda_recurrent_step_conv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, f, vp, vp, vp, i,
                                            i, vp]
    lib.kda_recurrent_step_conv.restype = ctypes.c_int
    for name in ("kda_recurrent_step_bwd_f32", "kda_recurrent_step_bwd"):
        fn = getattr(lib, name)
        fn.argtypes = [vp] * 5 + [f] + [vp] * 8 + [i, i, vp]
        fn.restype = ctypes.c_int
    for name in ("kda_chunk_bwd_f32", "kda_chunk_bwd"):
        fn = getattr(lib, name)
        fn.argtypes = [vp] * 5 + [f] + [vp] * 9 + [i, i, i, vp]
        fn.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_trim_workspace.argtypes = []
    lib.kda_trim_workspace.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().kda_status_string(int(status)).decode()


def trim_workspace() -> None:
    """Hand the library's cached workspace memory back to the driver (call
    when none of its work is in flight)."""
    st = load().kda_trim_workspace()
    if st != KDA_OK:
        raise KDAError(st, "kda_trim_workspace")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtype, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def chunk_fwd(q, k, v, g, beta, scale, h0=None, out=None, hT=None, final_state=True):
    """Chunkwise prefill.  q, k, v: [B, T, H, 128] bf16 (or all fp32 for the
    fp32 mode); g: [B, T, H, 128] fp32, or bf16 with bf16 q / k / v
    (kda_chunk_fwd_g16); beta: [B, T, H] fp32; h0: optional [B, H, 128, 128]
    fp32.  Returns (out, hT); hT is None when final_state is False and no hT
    buffer is given."""
    if q.dim() != 4 or q.shape[-1] != HEAD_DIM:
        raise ValueError(f"q: expected [B, T, H, {HEAD_DIM}], got {tuple(q.shape)}")
    B, T, H, _ = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda tensors must live on a GPU")
    io = q.dtype
    if io not in (torch.bfloat16, torch.float32):
        raise TypeError(f"q: dtype {io} not supported")
    for name, t in (("k", k), ("v", v)):
        _check(t, name, q.shape, io, dev)
    _check(q, "q", q.shape, io, dev)
    g16 = io == torch.bfloat16 and g.dtype == torch.bfloat16
    _check(g, "g", q.shape, torch.bfloat16 if g16 else torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    sshape = (B, H, HEAD_DIM, HEAD_DIM)
    if h0 is not None:
        _check(h0, "h0", sshape, torch.float32, dev)
    if out is None:
        out = torch.empty_like(v)
    else:
        _check(out, "out", q.shape, io, dev)
    if hT is None and final_state:
        hT = torch.empty(sshape, dtype=torch.float32, device=dev)
    elif hT is not None:
        _check(hT, "hT", sshape, torch.float32, dev)
    lib = load()
    fn = (lib.kda_chunk_fwd_g16 if g16 else lib.kda_chunk_fwd) if io == torch.bfloat16 \
        else lib.kda_chunk_fwd_f32
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(h0),
            _ptr(out), _ptr(hT), B, T, H, _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd")
    return out, hT


def chunk_fwd_noalloc(q, k, v, g, beta, scale, h0, out, hT=None):
    """kda_chunk_fwd_noalloc: the bf16 prefill with its workspace in the
    library's fixed per-GPU scratch, for callers that cannot allocate.  Every
    buffer is the caller's: q, k, v [B, T, H, 128] bf16, g [B, T, H, 128] fp32,
    beta [B, T, H] fp32, h0 and hT [B, H, 128, 128] fp32 or None, out like v.
    Returns (out, hT)."""
    B, T, H, _ = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check(t, name, q.shape, torch.bfloat16, dev)
    _check(g, "g", q.shape, torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    for name, t in (("h0", h0), ("hT", hT)):
        if t is not None:
            _check(t, name, (B, H, HEAD_DIM, HEAD_DIM), torch.float32, dev)
    st = load().kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      float(scale), _ptr(h0), _ptr(out), _ptr(hT), B, T, H,
                                      _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd_noalloc")
    return out, hT


def chunk_fwd_conv(q, k, v, wq, wk, wv, g, beta, scale, h0=None, conv_in=None,
                   conv_out=None, out=None, hT=None, final_state=True, final_conv=True,
                   gate=None):
    """Chunkwise prefill with the 4-tap short convolution + SiLU applied to the
    raw q, k, v first (kda_chunk_fwd_conv).  q, k, v: [B, T, H, 128] bf16 raw
    values; wq, wk, wv: [H, 128, 4] fp32 taps; conv_in / conv_out: optional
    [3, B, 3, H, 128] bf16 (q, k, v; the 3 raw tokens before the first, oldest
    first); gate: optional [B, T, H, 128] bf16 logits of the output gate (out =
    o * sigmoid(gate)); the rest as chunk_fwd with fp32 g.  Returns (out, hT,
    conv_out); conv_out is None when final_conv is False and no buffer is
    given."""
    if q.dim() != 4 or q.shape[-1] != HEAD_DIM:
        raise ValueError(f"q: expected [B, T, H, {HEAD_DIM}], got {tuple(q.shape)}")
    B, T, H, _ = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda tensors must live on a GPU")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, q.shape, torch.bfloat16, dev)
    for name, t in (("wq", wq), ("wk", wk), ("wv", wv)):
        _check(t, name, (H, HEAD_DIM, 4), torch.float32, dev)
    _check(g, "g", q.shape, torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    sshape = (B, H, HEAD_DIM, HEAD_DIM)
    cshape = (3, B, 3, H, HEAD_DIM)
    if h0 is not None:
        _check(h0, "h0", sshape, torch.float32, dev)
    if conv_in is not None:
        _check(conv_in, "conv_in", cshape, torch.bfloat16, dev)
    if gate is not None:
        _check(gate, "gate", q.shape, torch.bfloat16, dev)
    if out is None:
        out = torch.empty_like(v)
    else:
        _check(out, "out", q.shape, torch.bfloat16, dev)
    if hT is None and final_state:
        hT = torch.empty(sshape, dtype=torch.float32, device=dev)
    elif hT is not None:
        _check(hT, "hT", sshape, torch.float32, dev)
    if conv_out is None and final_conv:
        conv_out = torch.empty(cshape, dtype=torch.bfloat16, device=dev)
    elif conv_out is not None:
        _check(conv_out, "conv_out", cshape, torch.bfloat16, dev)
    st = load().kda_chunk_fwd_conv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(conv_in), _ptr(conv_out),
        _ptr(g), _ptr(beta), float(scale), _ptr(h0), _ptr(gate), _ptr(out), _ptr(hT), B, T, H,
        _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_chunk_fwd_conv")
    return out, hT, conv_out


def recurrent_step(q, k, v, g, beta, scale, S, out=None):
    """One decode step.  q, k, v: [B, H, 128] bf16 (or fp32); g: [B, H, 128]
    fp32; beta: [B, H] fp32; S: [B, H, 128, 128] fp32, updated in place.
    Returns out [B, H, 128]."""
    if q.dim() != 3 or q.shape[-1] != HEAD_DIM:
        raise ValueError(f"q: expected [B, H, {HEAD_DIM}], got {tuple(q.shape)}")
    B, H, _ = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda tensors must live on a GPU")
    io = q.dtype
    if io not in (torch.bfloat16, torch.float32):
        raise TypeError(f"q: dtype {io} not supported")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, q.shape, io, dev)
    _check(g, "g", q.shape, torch.float32, dev)
    _check(beta, "beta", (B, H), torch.float32, dev)
    _check(S, "S", (B, H, HEAD_DIM, HEAD_DIM), torch.float32, dev)
    if out is None:
        out = torch.empty_like(v)
    else:
        _check(out, "out", q.shape, io, dev)
    fn = load().kda_recurrent_step if io == torch.bfloat16 else load().kda_recurrent_step_f32
    st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(S), _ptr(out),
            B, H, _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_recurrent_step")
    return out


def recurrent_step_conv(q, k, v, wq, wk, wv, conv_state, g, beta, scale, S, out=None,
                        gate=None):
    """One decode step with the short convolution + SiLU on the raw q, k, v
    (kda_recurrent_step_conv).  q, k, v: [B, H, 128] bf16 raw values; wq, wk,
    wv: [H, 128, 4] fp32 taps; conv_state: [3, B, 3, H, 128] bf16 (the layout
    chunk_fwd_conv returns as conv_out), advanced in place; gate: optional
    [B, H, 128] bf16 logits of the output gate; g, beta, S as recurrent_step.
    Returns out [B, H, 128] bf16."""
    if q.dim() != 3 or q.shape[-1] != HEAD_DIM:
        raise ValueError(f"q: expected [B, H, {HEAD_DIM}], got {tuple(q.shape)}")
    B, H, _ = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda tensors must live on a GPU")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(t, name, q.shape, torch.bfloat16, dev)
    for name, t in (("wq", wq), ("wk", wk), ("wv", wv)):
        _check(t, name, (H, HEAD_DIM, 4), torch.float32, dev)
    _check(conv_state, "conv_state", (3, B, 3, H, HEAD_DIM), torch.bfloat16, dev)
    _check(g, "g", q.shape, torch.float32, dev)
    _check(beta, "beta", (B, H), torch.float32, dev)
    _check(S, "S", (B, H, HEAD_DIM, HEAD_DIM), torch.float32, dev)
    if gate is not None:
        _check(gate, "gate", q.shape, torch.bfloat16, dev)
    if out is None:
        out = torch.empty_like(v)
    else:
        _check(out, "out", q.shape, torch.bfloat16, dev)
    st = load().kda_recurrent_step_conv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(conv_state), _ptr(g),
        _ptr(beta), float(scale), _ptr(S), _ptr(gate), _ptr(out), B, H, _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_recurrent_step_conv")
    return out


def recurrent_step_bwd(q, k, v, g, beta, scale, S_prev, dout, dS):
    """Backward of one recurrent step (kda_recurrent_step_bwd_f32, or
    kda_recurrent_step_bwd for bf16 q / k / v / dout).  q, k, v, dout:
    [B, H, 128] fp32 or bf16 (all alike); g: [B, H, 128] fp32; beta: [B, H]
    fp32; S_prev: the state before the step; dS: [B, H, 128, 128] fp32
    gradient of the state after the step, replaced in place by the gradient
    of the state before it.  Returns (dq, dk, dv in the type of q, dg, dbeta
    fp32)."""
    if q.dim() != 3 or q.shape[-1] != HEAD_DIM:
        raise ValueError(f"q: expected [B, H, {HEAD_DIM}], got {tuple(q.shape)}")
    B, H, _ = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda tensors must live on a GPU")
    io = q.dtype
    if io not in (torch.bfloat16, torch.float32):
        raise TypeError(f"q: dtype {io} not supported")
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check(t, name, q.shape, io, dev)
    _check(g, "g", q.shape, torch.float32, dev)
    _check(beta, "beta", (B, H), torch.float32, dev)
    sshape = (B, H, HEAD_DIM, HEAD_DIM)
    _check(S_prev, "S_prev", sshape, torch.float32, dev)
    _check(dS, "dS", sshape, torch.float32, dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    dg = torch.empty_like(g)
    dbeta = torch.empty_like(beta)
    lib = load()
    fn = lib.kda_recurrent_step_bwd_f32 if io == torch.float32 else lib.kda_recurrent_step_bwd
    st = fn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(S_prev), _ptr(dout),
        _ptr(dS), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), B, H, _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, "kda_recurrent_step_bwd_f32")
    return dq, dk, dv, dg, dbeta


def chunk_bwd(q, k, v, g, beta, scale, dout, h0=None, dhT=None):
    """Backward of the chunked prefill (kda_chunk_bwd_f32, or kda_chunk_bwd for
    bf16 q / k / v / dout): gradients of <dout, o> + <dhT, hT> for (o, hT) =
    chunk_fwd(q, k, v, g, beta, scale, h0).  q, k, v, dout: [B, T, H, 128]
    fp32 or bf16 (all alike); g: [B, T, H, 128] fp32; beta: [B, T, H] fp32;
    h0, dhT: optional [B, H, 128, 128] fp32.  Returns (dq, dk, dv in the type
    of q, dg, dbeta, dh0 fp32)."""
    if q.dim() != 4 or q.shape[-1] != HEAD_DIM:
        raise ValueError(f"q: expected [B, T, H, {HEAD_DIM}], got {tuple(q.shape)}")
    B, T, H, _ = q.shape
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda tensors must live on a GPU")
    io = q.dtype
    if io not in (torch.bfloat16, torch.float32):
        raise TypeError(f"q: dtype {io} not supported")
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check(t, name, q.shape, io, dev)
    _check(g, "g", q.shape, torch.float32, dev)
    _check(beta, "beta", (B, T, H), torch.float32, dev)
    sshape = (B, H, HEAD_DIM, HEAD_DIM)
    if h0 is not None:
        _check(h0, "h0", sshape, torch.float32, dev)
    if dhT is not None:
        _check(dhT, "dhT", sshape, torch.float32, dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    dg = torch.empty_like(g)
    dbeta = torch.empty_like(beta)
    dh0 = torch.empty(sshape, dtype=torch.float32, device=dev)
    lib = load()
    name = "kda_chunk_bwd_f32" if io == torch.float32 else "kda_chunk_bwd"
    st = getattr(lib, name)(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(h0), _ptr(dout),
        _ptr(dhT), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0), B, T, H,
        _stream(dev))
    if st != KDA_OK:
        raise KDAError(st, name)
    return dq, dk, dv, dg, dbeta, dh0
