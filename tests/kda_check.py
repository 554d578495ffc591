"""Shared helpers for the GPU parity tests: run the fp64 oracle on the exact
bytes the GPU consumed, and the error metrics the tolerances are stated in.

Metrics (per (batch, head), worst one reported):
  output : max_{t,j} |o - o_ref| / max_{t,j} |o_ref|
  state  : max_{i,j} |S - S_ref| / max_{i,j} |S_ref|
"""
import os

import numpy as np
import torch

from oracle import oracle

# max|o - o_ref| / max|o_ref| for bf16 inputs, and the final-state bound in
# fp32-input mode; the bf16 state bound is taken equal to the bf16 output bound.
TOL_BF16 = 1e-2
TOL_F32 = 1e-3


def host64(t):
    return t.detach().to("cpu").double().numpy()


def oracle_threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 4


def oracle_prefill(inp, heads=None, t_slice=None):
    """Oracle on the GPU tensors in ``inp`` (q, k, v, g, beta [, h0], scale),
    optionally restricted to some heads.  Returns (o, hT) as float64 arrays
    in [B, T, Hs, D] and [B, Hs, D, D]."""
    sel = slice(None) if heads is None else list(heads)
    ts = slice(None) if t_slice is None else t_slice

    def pick(x):
        return host64(x[:, ts][:, :, sel])

    h0 = inp.get("h0")
    h0 = None if h0 is None else host64(h0[:, sel])
    return oracle.forward(pick(inp["q"]), pick(inp["k"]), pick(inp["v"]), pick(inp["g"]),
                          host64(inp["beta"][:, ts][:, :, sel]), inp["scale"], h0,
                          threads=oracle_threads())


def rel_out(o, ref):
    """Worst per-(b, h) normalised max error; o and ref are [B, T, H, D]."""
    o = np.asarray(o, dtype=np.float64)
    err = np.abs(o - ref).max(axis=(1, 3))
    den = np.abs(ref).max(axis=(1, 3))
    return float((err / np.where(den > 0, den, 1.0)).max())


def rel_state(s, ref):
    """Worst per-(b, h) normalised max error; s and ref are [B, H, D, D]."""
    s = np.asarray(s, dtype=np.float64)
    err = np.abs(s - ref).max(axis=(2, 3))
    den = np.abs(ref).max(axis=(2, 3))
    return float((err / np.where(den > 0, den, 1.0)).max())


def say(msg):
    print(msg, flush=True)
