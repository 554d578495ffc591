"""Test infrastructure only: a second, matrix-form statement of the KDA
recurrence, used to pin the C oracle (it shares no code with it).

One token of the recurrence (Kimi-K3 深度解析 blog, section 三: decay per
channel, then add the error ``beta (v - vhat)`` along the key, ``vhat`` read
from the decayed state) is an affine map of the state.  With the state stored
key-channel-major (``S`` is ``Dk x Dv``) and ``kh`` the unit key,

    S_t = M_t S_{t-1} + beta_t kh_t v_t^T,
    M_t = (I - beta_t kh_t kh_t^T) Diag(exp g_t),

so after T tokens

    S_T = M_T ... M_1 S_0 + sum_t M_T ... M_{t+1} beta_t kh_t v_t^T,

and the read-out is ``o_t = scale S_t^T qh_t``.  Here every ``M_t`` is built as
an explicit ``Dk x Dk`` matrix and the products are formed with ``@``; nothing
is computed row by row as in the oracle.  Meant for T <= 8.
"""
from __future__ import annotations

import numpy as np


def _unit(x, eps):
    return x / np.sqrt(np.sum(x * x) + eps)


def transition_matrices(k, g, beta, eps=1e-6):
    """Per-token ``M_t`` and the injected term's key vector ``beta_t kh_t``.
    k, g: [T, Dk]; beta: [T]."""
    T, dk = k.shape
    eye = np.eye(dk)
    Ms, ws = [], []
    for t in range(T):
        kh = _unit(np.asarray(k[t], dtype=np.float64), eps)
        Ms.append((eye - beta[t] * np.outer(kh, kh)) @ np.diag(np.exp(g[t])))
        ws.append(beta[t] * kh)
    return Ms, ws


def run(q, k, v, g, beta, scale, S0=None, eps=1e-6):
    """One sequence: q, k, g [T, Dk]; v [T, Dv]; beta [T]; S0 [Dk, Dv].
    Returns (o [T, Dv], S_T) built from products of materialised M_t."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64)
    Ms, ws = transition_matrices(k, g, beta, eps)
    o = np.zeros((T, dv))
    for t in range(T):
        # S_t from scratch: the full product applied to S0 plus every injection
        prod = np.eye(dk)
        for s in range(t, -1, -1):
            prod = prod @ Ms[s]
        St = prod @ S0
        for s in range(t + 1):
            tail = np.eye(dk)
            for r in range(t, s, -1):
                tail = tail @ Ms[r]
            St = St + tail @ np.outer(ws[s], v[s])
        o[t] = scale * (St.T @ _unit(q[t], eps))
    return o, St if T > 0 else S0
