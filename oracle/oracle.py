"""Test infrastructure only: Python side of the fp64 CPU oracle.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg import
this module.  The GPU library never does, and nothing here imports the GPU
library: the two share no code.

``forward`` runs the token-by-token Kimi Delta Attention recurrence in
``kda_oracle.c`` (decay the state per key channel, predict the value for the
normalised key from the decayed state, write the scaled error along the key,
read out with the normalised query; Kimi-K3 深度解析 blog, section 三, and the
KDA paragraph of the 深入 Kimi-K3 thread for the in-kernel L2 normalisation and
the per-channel decay).  Inputs are widened to float64 from whatever exact
values the caller holds (for GPU parity: the very bf16/fp32 bytes the GPU
consumed), so input quantisation never counts as error.

``step_backward`` is the reverse-mode derivative of one recurrent step and
``sequence_backward`` that of the whole recurrence, token by token in reverse
over the kept states (in ``kda_oracle.c``); both are pinned to central
differences of ``forward``.  ``chunk_backward`` differentiates the chunkwise
form instead; it is kept as a CPU cross-check of that algebra, pinned to the
token-by-token backward, and is not the reference of any GPU comparison.

Layouts follow the library's: q, k, v, g, o are ``[B, T, H, D]``; beta is
``[B, T, H]``; h0 and hT are ``[B, H, Dk, Dv]`` (key channel = row).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "_kda_oracle.so")
_lib = None


def build() -> str:
    """Compile the C oracle with gcc (always; cheap)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O3", "-std=c99", "-Wall", "-shared", "-fPIC", "-pthread",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    _lib = configure(ctypes.CDLL(_LIB))
    return _lib


def configure(lib):
    """Declares the C entry points' signatures on a loaded oracle library
    (this one, or a copy built from a modified source by a test)."""
    dp = ctypes.POINTER(ctypes.c_double)
    lib.kda_oracle_run.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        dp, dp, dp, dp, dp, ctypes.c_double, ctypes.c_double, dp, dp, dp,
        ctypes.c_int]
    lib.kda_oracle_run.restype = ctypes.c_int
    lib.kda_oracle_seq_backward.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        dp, dp, dp, dp, dp, ctypes.c_double, ctypes.c_double, dp, dp, dp,
        dp, dp, dp, dp, dp, dp, ctypes.c_int]
    lib.kda_oracle_seq_backward.restype = ctypes.c_int
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(x):
    """Widen to a C-contiguous float64 numpy array (accepts torch tensors)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: widen exactly, then hand over
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def run_sequences(q, k, v, g, beta, scale, h0=None, eps=1e-6, threads=None):
    """Sequence-major entry: q, k, g ``[N, T, Dk]``; v ``[N, T, Dv]``;
    beta ``[N, T]``; h0 ``[N, Dk, Dv]`` or None.  Returns (o, hT)."""
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    n, T, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (n, T, dk) and g.shape == (n, T, dk)
    assert v.shape == (n, T, dv) and beta.shape == (n, T)
    if h0 is not None:
        assert h0.shape == (n, dk, dv)
    o = np.zeros((n, T, dv), dtype=np.float64)
    hT = np.zeros((n, dk, dv), dtype=np.float64)
    rc = _load().kda_oracle_run(
        n, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        float(scale), float(eps), _ptr(h0), _ptr(o), _ptr(hT),
        int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_run failed with {rc}")
    return o, hT


def forward(q, k, v, g, beta, scale, h0=None, eps=1e-6, threads=None):
    """Library layout entry: q, k, v, g ``[B, T, H, D]``, beta ``[B, T, H]``,
    h0 ``[B, H, Dk, Dv]`` or None.  Returns (o ``[B, T, H, Dv]``, hT)."""
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    B, T, H, dk = q.shape
    dv = v.shape[3]

    def seq(x):  # [B, T, H, D] -> [B*H, T, D]
        return np.ascontiguousarray(x.transpose(0, 2, 1, 3).reshape(B * H, T, -1))

    o, hT = run_sequences(
        seq(q), seq(k), seq(v), seq(g),
        np.ascontiguousarray(beta.transpose(0, 2, 1).reshape(B * H, T)),
        scale, None if h0 is None else h0.reshape(B * H, dk, dv), eps, threads)
    o = o.reshape(B, H, T, dv).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(o), hT.reshape(B, H, dk, dv)


def step(q, k, v, g, beta, scale, S, eps=1e-6, threads=None):
    """One decode step: q, k, v, g ``[B, H, D]``, beta ``[B, H]``,
    S ``[B, H, Dk, Dv]``.  Returns (o ``[B, H, Dv]``, S_new)."""
    q, k, v, g, beta, S = map(_f64, (q, k, v, g, beta, S))
    B, H, dk = q.shape
    dv = v.shape[2]
    o, hT = run_sequences(
        q.reshape(B * H, 1, dk), k.reshape(B * H, 1, dk), v.reshape(B * H, 1, dv),
        g.reshape(B * H, 1, dk), beta.reshape(B * H, 1), scale,
        S.reshape(B * H, dk, dv), eps, threads)
    return o.reshape(B, H, dv), hT.reshape(B, H, dk, dv)


# ---------------------------------------------------------------------------
# Short convolution in front of the attention (the KDA paragraph of the
# 深入 Kimi-K3 thread: q, k and v each pass through a short convolution with
# SiLU before the kernel; the Kimi K3 architecture page's config table: a
# kernel of 4 taps).  Read here as the plainest form those passages support:
# depthwise (one 4-tap filter per head and channel), causal, no bias, SiLU on
# the filtered value, and a state of the 3 raw tokens that precede the first
# one (zeros for a fresh sequence).
# ---------------------------------------------------------------------------
CONV_TAPS = 4


def silu(x):
    """x * logistic(x), in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def round_bf16(x):
    """x rounded to fp32 and then to bf16, each to nearest with ties to even,
    returned as fp64: the bf16 value an fp32 computation of x stores (finite
    x only)."""
    bits = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32)).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    r = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32).astype(np.float64)


def short_conv_silu(x, w, state=None, round_out=False):
    """x ``[B, T, H, D]`` raw values; w ``[H, D, 4]`` taps, tap j weighting
    the token j - 3 steps from the current one (tap 3 = the current token);
    state ``[B, 3, H, D]`` the raw tokens before x (oldest first) or None for
    zeros.  Returns (y ``[B, T, H, D]`` = silu(sum_j w_j x_{t-3+j}), the new
    state: the last 3 raw tokens of state followed by x).  round_out: y is
    rounded to bf16 (round_bf16), the type in which a bf16 attention takes
    its q, k and v."""
    x, w = _f64(x), _f64(w)
    B, T, H, D = x.shape
    assert w.shape == (H, D, CONV_TAPS)
    prev = np.zeros((B, CONV_TAPS - 1, H, D)) if state is None else _f64(state)
    assert prev.shape == (B, CONV_TAPS - 1, H, D)
    full = np.concatenate([prev, x], axis=1)  # token t of x sits at index t + 3
    pre = np.zeros((B, T, H, D))
    for j in range(CONV_TAPS):
        pre += w[None, None, :, :, j] * full[:, j:j + T]
    y = silu(pre)
    return (round_bf16(y) if round_out else y), np.ascontiguousarray(full[:, T:])


def output_gate(o, z):
    """The output gate behind the attention: o * sigmoid(z) elementwise, z the
    gate's logits (one per output channel: the thread's full-rank gate, read
    as the sigmoid gate it names for the global layers)."""
    return _f64(o) / (1.0 + np.exp(-_f64(z)))


def forward_conv(q, k, v, wq, wk, wv, g, beta, scale, h0=None, conv_state=None, eps=1e-6,
                 threads=None, round_bf16_inputs=False, gate=None):
    """The attention on the short-convolved q, k, v.  conv_state is None or a
    triple of ``[B, 3, H, D]`` states for q, k, v.  round_bf16_inputs: the
    filtered q, k, v are rounded to bf16 before the attention.  gate: None or
    the ``[B, T, H, D]`` logits of the output gate.  Returns (o, hT, the three
    new conv states)."""
    cs = (None, None, None) if conv_state is None else conv_state
    r = round_bf16_inputs
    qc, sq = short_conv_silu(q, wq, cs[0], r)
    kc, sk = short_conv_silu(k, wk, cs[1], r)
    vc, sv = short_conv_silu(v, wv, cs[2], r)
    o, hT = forward(qc, kc, vc, g, beta, scale, h0, eps, threads)
    if gate is not None:
        o = output_gate(o, gate)
    return o, hT, (sq, sk, sv)


def step_conv(q, k, v, wq, wk, wv, conv_state, g, beta, scale, S, eps=1e-6, threads=None,
              round_bf16_inputs=False, gate=None):
    """One decode token of the attention on the short-convolved q, k, v: the
    filter of short_conv_silu applied to the single new token ``[B, H, D]``
    with the carried conv states (a triple of ``[B, 3, H, D]``: the raw tokens
    before it, oldest first), then one step of the recurrence.
    round_bf16_inputs and gate (``[B, H, D]``) as forward_conv.  Returns (o,
    new S, the three new conv states)."""
    ys, states = [], []
    for x, w, st in ((q, wq, conv_state[0]), (k, wk, conv_state[1]), (v, wv, conv_state[2])):
        y, ns = short_conv_silu(_f64(x)[:, None], w, st, round_bf16_inputs)
        ys.append(y[:, 0])
        states.append(ns)
    o, S_new = step(ys[0], ys[1], ys[2], g, beta, scale, S, eps, threads)
    if gate is not None:
        o = output_gate(o, gate)
    return o, S_new, tuple(states)


# ---------------------------------------------------------------------------
# Backward of one recurrent step (training through the recurrence, one token
# at a time in reverse).  The pages say only that the log-decay bound serves
# training speed (the ai-pulse-lab summary of the technical report, KDA
# paragraph); the gradient is derived here by reverse-mode differentiation of
# the step's own assignments, in reverse order.
# ---------------------------------------------------------------------------
def step_backward(q, k, v, g, beta, scale, S_prev, d_o, dS_next, eps=1e-6):
    """Gradients of L = sum(d_o * o) + sum(dS_next * S_new) for one step
    S_new, o = step(q, k, v, g, beta, scale, S_prev).  Shapes as ``step``
    (d_o like o, dS_next like S).  Returns (dq, dk, dv, dg, dbeta, dS_prev)
    in fp64, one (b, h) at a time with plain numpy."""
    q, k, v, g, beta, S_prev, d_o, dS_next = map(
        _f64, (q, k, v, g, beta, S_prev, d_o, dS_next))
    dq, dk, dv, dg = (np.zeros_like(x) for x in (q, k, v, g))
    dbeta = np.zeros_like(beta)
    dS_prev = np.zeros_like(S_prev)
    B, H = q.shape[:2]
    for b in range(B):
        for h in range(H):
            # forward, keeping every intermediate
            rq = 1.0 / np.sqrt(q[b, h] @ q[b, h] + eps)
            rk = 1.0 / np.sqrt(k[b, h] @ k[b, h] + eps)
            qh, kh = q[b, h] * rq, k[b, h] * rk
            a = np.exp(g[b, h])
            St = a[:, None] * S_prev[b, h]           # decayed state
            p = St.T @ kh                              # prediction
            bt = beta[b, h]
            u = bt * (v[b, h] - p)                     # scaled error
            Sn = St + np.outer(kh, u)                  # new state
            # o = scale * Sn^T qh
            G = dS_next[b, h] + scale * np.outer(qh, d_o[b, h])   # dL/dSn
            dqh = scale * (Sn @ d_o[b, h])
            # Sn = St + kh u^T
            dSt = G.copy()
            dkh = G @ u
            du = G.T @ kh
            # u = beta (v - p)
            dv[b, h] = bt * du
            dbeta[b, h] = du @ (v[b, h] - p)
            dp = -bt * du
            # p = St^T kh
            dSt += np.outer(kh, dp)
            dkh += St @ dp
            # St = diag(exp g) S_prev
            dS_prev[b, h] = a[:, None] * dSt
            dg[b, h] = np.sum(St * dSt, axis=1)
            # qh = q / sqrt(|q|^2 + eps), likewise k
            dq[b, h] = rq * dqh - rq ** 3 * (q[b, h] @ dqh) * q[b, h]
            dk[b, h] = rk * dkh - rk ** 3 * (k[b, h] @ dkh) * k[b, h]
    return dq, dk, dv, dg, dbeta, dS_prev


def sequence_backward(q, k, v, g, beta, scale, h0, d_o, d_hT=None, eps=1e-6, threads=None):
    """Gradients of L = <d_o, o> + <d_hT, hT> for (o, hT) = forward(q, k, v,
    g, beta, scale, h0): the recurrence run forward keeping the state before
    every token, then every token's assignments differentiated in reverse
    order (kda_oracle_seq_backward in kda_oracle.c), exactly the chain of
    ``step_backward`` over the sequence.  Library layout as ``forward``; h0
    and d_hT may be None (zeros).  Returns (dq, dk, dv, dg, dbeta, dh0) in
    fp64.  Each thread keeps T + 1 states of one sequence: (T + 1) * Dk * Dv
    doubles."""
    q, k, v, g, beta, h0, d_o, d_hT = map(_f64, (q, k, v, g, beta, h0, d_o, d_hT))
    B, T, H, dk = q.shape
    dv = v.shape[3]

    def seq(x):  # [B, T, H, D] -> [B*H, T, D]
        return np.ascontiguousarray(x.transpose(0, 2, 1, 3).reshape(B * H, T, x.shape[3]))

    def unseq(x):  # [B*H, T, D] -> [B, T, H, D]
        return np.ascontiguousarray(x.reshape(B, H, T, x.shape[2]).transpose(0, 2, 1, 3))

    n = B * H
    gq, gk, gv, gg = (np.zeros((n, T, d)) for d in (dk, dk, dv, dk))
    gb = np.zeros((n, T))
    dh0 = np.zeros((n, dk, dv))
    st = lambda x: None if x is None else np.ascontiguousarray(x.reshape(n, dk, dv))
    rc = _load().kda_oracle_seq_backward(
        n, T, dk, dv, _ptr(seq(q)), _ptr(seq(k)), _ptr(seq(v)), _ptr(seq(g)),
        _ptr(np.ascontiguousarray(beta.transpose(0, 2, 1).reshape(n, T))), float(scale),
        float(eps), _ptr(st(h0)), _ptr(seq(d_o)), _ptr(st(d_hT)), _ptr(gq), _ptr(gk), _ptr(gv),
        _ptr(gg), _ptr(gb), _ptr(dh0), int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_seq_backward failed with {rc}")
    dbeta = np.ascontiguousarray(gb.reshape(B, H, T).transpose(0, 2, 1))
    return unseq(gq), unseq(gk), unseq(gv), unseq(gg), dbeta, dh0.reshape(B, H, dk, dv)


# ---------------------------------------------------------------------------
# Backward of the chunkwise prefill.  The chunk form (derived from the
# recurrence, not printed on the pages): for a chunk of tokens r = 0..C-1
# entering with state S, with Gam_r = sum_{s<=r} g_s per channel and L the
# chunk's last token,
#   Kt_r = e^{Gam_r} kh_r, Qt_r = e^{Gam_r} qh_r, Kb_r = e^{Gam_L - Gam_r} kh_r,
#   gamma = e^{Gam_L},
#   P_ri = sum_c kh_rc kh_ic e^{Gam_rc - Gam_ic} (i < r),  A = diag(beta) P,
#   N_ri = sum_c qh_rc kh_ic e^{Gam_rc - Gam_ic} (i <= r),  M = N,
#   X = (I + A)^-1,  T = X diag(beta),  R = V - Kt S,  U = T R,
#   O = scale (Qt S + M U),  S' = Diag(gamma) S + Kb^T U.
# Its reverse-mode derivative, assignment by assignment in reverse order, is
# written out below in fp64 (no factorisation of the decays is needed at
# this precision: e^{+-320} is finite in fp64).
# ---------------------------------------------------------------------------
def _chunk_backward_one(qh, kh, v, g, beta, scale, S, dO, dSn):
    """One chunk of one (b, h): qh, kh [C, Dk] normalised, v [C, Dv], g [C,
    Dk], beta [C], S [Dk, Dv] entering state, dO [C, Dv], dSn = dL/dS'.
    Returns (dqh, dkh, dv, dg, dbeta, dS)."""
    C = qh.shape[0]
    Gam = np.cumsum(g, axis=0)
    GL = Gam[-1]
    eG = np.exp(Gam)
    Kt, Qt = eG * kh, eG * qh
    eB = np.exp(GL[None, :] - Gam)
    Kb = eB * kh
    gam = np.exp(GL)
    E = np.exp(Gam[:, None, :] - Gam[None, :, :])            # [r, i, c]
    P = np.einsum("rc,ic,ric->ri", kh, kh, E)
    N = np.einsum("rc,ic,ric->ri", qh, kh, E)
    strict = np.tril(np.ones((C, C)), -1)
    incl = np.tril(np.ones((C, C)))
    A = beta[:, None] * P * strict
    M = N * incl
    X = np.linalg.inv(np.eye(C) + A)
    T = X * beta[None, :]
    R = v - Kt @ S
    U = T @ R
    # reverse
    dU = scale * M.T @ dO + Kb @ dSn
    dM = scale * (dO @ U.T) * incl
    dQt = scale * dO @ S.T
    dKb = U @ dSn.T
    dgam = np.sum(dSn * S, axis=1)
    dT = (dU @ R.T) * incl
    dR = T.T @ dU
    dv = dR
    dKt = -dR @ S.T
    dS = scale * Qt.T @ dO + gam[:, None] * dSn - Kt.T @ dR
    dX = dT * beta[None, :]
    dbeta = np.sum(X * dT, axis=0)
    dA = -(X.T @ dX @ X.T) * strict
    dbeta = dbeta + np.sum(dA * P, axis=1)
    dP = beta[:, None] * dA
    dN = dM
    dkh = np.zeros_like(kh)
    dqh = np.zeros_like(qh)
    dGam = np.zeros_like(Gam)
    # P_ri = sum_c kh_rc kh_ic E_ric ; N_ri = sum_c qh_rc kh_ic E_ric
    wP = dP[:, :, None] * E                                 # [r, i, c]
    wN = dN[:, :, None] * E
    dkh += np.einsum("ric,ic->rc", wP, kh) + np.einsum("ric,rc->ic", wP, kh)
    dqh += np.einsum("ric,ic->rc", wN, kh)
    dkh += np.einsum("ric,rc->ic", wN, qh)
    tP = wP * kh[:, None, :] * kh[None, :, :]
    tN = wN * qh[:, None, :] * kh[None, :, :]
    dGam += tP.sum(axis=1) - tP.sum(axis=0) + tN.sum(axis=1) - tN.sum(axis=0)
    # Kt, Qt, Kb, gamma
    dkh += eG * dKt
    dGam += Kt * dKt
    dqh += eG * dQt
    dGam += Qt * dQt
    dkh += eB * dKb
    dGam -= Kb * dKb
    dGam[-1] += np.sum(Kb * dKb, axis=0) + gam * dgam
    # Gam_r = sum_{s <= r} g_s
    dg = np.cumsum(dGam[::-1], axis=0)[::-1]
    return dqh, dkh, dv, dg, dbeta, dS


def chunk_backward(q, k, v, g, beta, scale, h0, d_o, d_hT=None, chunk=64, eps=1e-6):
    """Gradients of L = <d_o, o> + <d_hT, hT> for (o, hT) = forward(q, k, v,
    g, beta, scale, h0), computed the chunkwise way: a forward pass keeps the
    state entering each chunk, then the chunks are differentiated in reverse
    (_chunk_backward_one), the state gradient carried from one to the one
    before.  Shapes as ``forward``; h0 may be None (zeros).  Returns (dq, dk,
    dv, dg, dbeta, dh0) in fp64."""
    q, k, v, g, beta, d_o = map(_f64, (q, k, v, g, beta, d_o))
    B, T, H, D = q.shape
    Dv = v.shape[3]
    h0 = np.zeros((B, H, D, Dv)) if h0 is None else _f64(h0)
    d_hT = np.zeros((B, H, D, Dv)) if d_hT is None else _f64(d_hT)
    dq, dk, dv, dg = (np.zeros_like(x) for x in (q, k, v, g))
    dbeta = np.zeros_like(beta)
    dh0 = np.zeros_like(h0)
    starts = list(range(0, T, chunk))
    for b in range(B):
        for h in range(H):
            rq = 1.0 / np.sqrt(np.sum(q[b, :, h] ** 2, axis=1) + eps)
            rk = 1.0 / np.sqrt(np.sum(k[b, :, h] ** 2, axis=1) + eps)
            qh, kh = q[b, :, h] * rq[:, None], k[b, :, h] * rk[:, None]
            # forward over the chunks, keeping each entering state
            S = h0[b, h].copy()
            states = []
            for c0 in starts:
                sl = slice(c0, min(T, c0 + chunk))
                states.append(S.copy())
                for r in range(sl.stop - sl.start):   # the recurrence within the chunk
                    t = sl.start + r
                    S = np.exp(g[b, t, h])[:, None] * S
                    u = beta[b, t, h] * (v[b, t, h] - S.T @ kh[t])
                    S = S + np.outer(kh[t], u)
            dS = d_hT[b, h].copy()
            dqh = np.zeros_like(qh)
            dkh = np.zeros_like(kh)
            for ci in reversed(range(len(starts))):
                sl = slice(starts[ci], min(T, starts[ci] + chunk))
                r = _chunk_backward_one(qh[sl], kh[sl], v[b, sl, h], g[b, sl, h],
                                        beta[b, sl, h], scale, states[ci], d_o[b, sl, h], dS)
                dqh[sl], dkh[sl] = r[0], r[1]
                dv[b, sl, h], dg[b, sl, h], dbeta[b, sl, h] = r[2], r[3], r[4]
                dS = r[5]
            dh0[b, h] = dS
            # qh = q / sqrt(|q|^2 + eps), likewise k
            dq[b, :, h] = rq[:, None] * dqh - (rq ** 3 * np.sum(q[b, :, h] * dqh, axis=1))[:, None] * q[b, :, h]
            dk[b, :, h] = rk[:, None] * dkh - (rk ** 3 * np.sum(k[b, :, h] * dkh, axis=1))[:, None] * k[b, :, h]
    return dq, dk, dv, dg, dbeta, dh0
