"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test fixes the oracle to something the pages or plain mathematics state:
a hand-derived worked example, the materialised product of per-token
transition matrices, closed forms of special cases (orthonormal recall, beta=1
exact recall, pure decay, pure read-out), structural invariants (chaining,
normalisation invariance, linearity) and the state-size arithmetic quoted by
the 深入 Kimi-K3 thread.  Everything here runs on the CPU.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle, transition_product as tp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, B, T, H, dk, dv, g_shift=4.0, with_h0=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g = -5.0 / (1.0 + np.exp(-(rng.standard_normal((B, T, H, dk)) - g_shift)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    h0 = rng.standard_normal((B, H, dk, dv)) * 0.1 if with_h0 else None
    return q, k, v, g, beta, h0


def _rel(a, b):
    den = np.abs(b).max()
    return np.abs(a - b).max() / (den if den > 0 else 1.0)


def test_golden_hand_example():
    """Hand-derived two-token example; catches decay on the wrong side, a
    prediction from the undecayed state, a read-out before the write and a
    dropped beta (each changes the printed numbers)."""
    with open(os.path.join(GOLDEN, "kda_tiny_hand.json")) as f:
        case = json.load(f)
    arr = lambda key: np.array(case[key], dtype=np.float64)
    q, k, v, g = (arr(x)[None, :, None, :] for x in ("q", "k", "v", "g"))
    beta = arr("beta")[None, :, None]
    o, hT = oracle.forward(q, k, v, g, beta, case["scale"], eps=case["eps"], threads=1)
    np.testing.assert_allclose(o[0, :, 0], arr("o"), rtol=0, atol=1e-15)
    np.testing.assert_allclose(hT[0, 0], arr("hT"), rtol=0, atol=1e-15)


@pytest.mark.parametrize("dk,dv,T", [(4, 3, 1), (8, 8, 5), (16, 12, 8), (128, 128, 6)])
def test_transition_product(dk, dv, T):
    """P1: the oracle equals the product of materialised per-token matrices
    M_t = (I - beta kh kh^T) Diag(exp g) applied to h0 plus the injections."""
    rng = np.random.default_rng(100 + dk + T)
    q, k, v, g, beta, h0 = _rand_case(rng, 1, T, 1, dk, dv)
    o, hT = oracle.forward(q, k, v, g, beta, 0.37, h0, threads=1)
    o2, hT2 = tp.run(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0],
                     0.37, h0[0, 0])
    assert _rel(o[0, :, 0], o2) < 1e-12
    assert _rel(hT[0, 0], hT2) < 1e-12


def test_transition_product_at_bound():
    """P1 with the decay at its lower bound (g = -5) and at 0, alternating."""
    rng = np.random.default_rng(7)
    T, d = 8, 32
    q, k, v, _, beta, h0 = _rand_case(rng, 1, T, 1, d, d)
    g = np.where((np.arange(T)[:, None] + np.arange(d)[None, :]) % 2 == 0, -5.0, 0.0)
    g = g[None, :, None, :]
    o, hT = oracle.forward(q, k, v, g, beta, 1.0, h0, threads=1)
    o2, hT2 = tp.run(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0],
                     1.0, h0[0, 0])
    assert _rel(o[0, :, 0], o2) < 1e-12
    assert _rel(hT[0, 0], hT2) < 1e-12


def _signed_basis_keys(rng, T, d):
    perm = rng.permutation(d)[:T]
    sign = rng.choice([-1.0, 1.0], size=T)
    keys = np.zeros((T, d))
    keys[np.arange(T), perm] = sign * rng.uniform(0.5, 3.0, size=T)  # any length
    return keys


def _hadamard(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("kind", ["basis", "hadamard"])
def test_orthonormal_recall(kind):
    """P2: with g = 0, beta = 1, h0 = 0 and mutually orthogonal keys the
    recurrence is plain linear attention over a key-value memory: a query equal
    to an earlier key returns scale * its value, and hT^T kh_j = v_j."""
    rng = np.random.default_rng(11)
    d, T = 64, 48
    if kind == "basis":
        keys = _signed_basis_keys(rng, T, d)
    else:
        keys = _hadamard(d)[rng.permutation(d)[:T]] * rng.uniform(0.5, 2.0, (T, 1))
    v = rng.standard_normal((T, d))
    pick = np.array([rng.integers(0, t + 1) for t in range(T)])
    q = keys[pick] * rng.uniform(0.2, 4.0, (T, 1))
    g = np.zeros((T, d))
    beta = np.ones(T)
    scale = 0.125
    o, hT = oracle.forward(q[None, :, None], keys[None, :, None], v[None, :, None],
                           g[None, :, None], beta[None, :, None], scale, eps=0.0, threads=1)
    np.testing.assert_allclose(o[0, :, 0], scale * v[pick], rtol=0, atol=1e-13)
    kh = keys / np.linalg.norm(keys, axis=1, keepdims=True)
    np.testing.assert_allclose(kh @ hT[0, 0], v, rtol=0, atol=1e-13)


@pytest.mark.parametrize("gmode", ["random", "bound", "zero"])
def test_beta_one_exact_recall(gmode):
    """P3: with beta = 1 every write makes S_t^T kh_t = v_t exactly, whatever
    the decay; with q_t = k_t the read-out is scale * v_t at every t."""
    rng = np.random.default_rng(12)
    T, d = 300, 128
    q, k, v, g, _, h0 = _rand_case(rng, 1, T, 1, d, d)
    if gmode == "bound":
        g = np.full_like(g, -5.0)
    elif gmode == "zero":
        g = np.zeros_like(g)
    beta = np.ones((1, T, 1))
    o, _ = oracle.forward(k, k, v, g, beta, 0.25, h0, eps=0.0, threads=1)
    np.testing.assert_allclose(o, 0.25 * v, rtol=0, atol=1e-12)


def test_beta_zero_pure_decay():
    """P4: with beta = 0 nothing is written: S_t = Diag(exp(sum_{s<=t} g_s)) h0
    (decay on key rows) and o_t = scale S_t^T qh_t."""
    rng = np.random.default_rng(13)
    B, T, H, dk, dv = 2, 40, 3, 16, 8
    q, k, v, g, _, h0 = _rand_case(rng, B, T, H, dk, dv)
    beta = np.zeros((B, T, H))
    eps = 1e-6
    o, hT = oracle.forward(q, k, v, g, beta, 0.5, h0, eps=eps, threads=2)
    G = np.cumsum(g, axis=1)  # [B, T, H, dk]
    qh = q / np.sqrt((q * q).sum(-1, keepdims=True) + eps)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                St = np.exp(G[b, t, h])[:, None] * h0[b, h]
                np.testing.assert_allclose(o[b, t, h], 0.5 * St.T @ qh[b, t, h],
                                           rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(hT[b, h], np.exp(G[b, -1, h])[:, None] * h0[b, h],
                                       rtol=1e-12, atol=1e-300)
    o0, hT0 = oracle.forward(q, k, v, g, beta, 0.5, None, threads=2)
    assert not o0.any() and not hT0.any()


def test_read_only():
    """P5: g = 0 and beta = 0 leave the state alone: o_t = scale h0^T qh_t."""
    rng = np.random.default_rng(14)
    B, T, H, dk, dv = 1, 20, 2, 32, 24
    q, k, v, _, _, h0 = _rand_case(rng, B, T, H, dk, dv)
    g = np.zeros((B, T, H, dk))
    beta = np.zeros((B, T, H))
    o, hT = oracle.forward(q, k, v, g, beta, 0.3, h0, eps=0.0, threads=1)
    qh = q / np.linalg.norm(q, axis=-1, keepdims=True)
    want = 0.3 * np.einsum("bthi,bhij->bthj", qh, h0)
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(hT, h0)


def test_state_size_invariants():
    """P6: the thread's figures for 69 KDA layers of 96 heads with 128x128
    fp32 states: about 1.09e8 values and about 434 MB per sequence, whatever
    the context length.  The oracle's final state has that per-layer shape for
    any T."""
    layers, heads, d = 69, 96, 128
    values = layers * heads * d * d
    assert values == 108_527_616 and round(values / 1e8, 2) == 1.09
    assert values * 4 == 434_110_464 and round(values * 4 / 1e6) == 434
    rng = np.random.default_rng(15)
    for T in (1, 7, 33):
        q, k, v, g, beta, _ = _rand_case(rng, 1, T, 2, d, d, with_h0=False)
        _, hT = oracle.forward(q, k, v, g, beta, 1.0, threads=2)
        assert hT.shape == (1, 2, d, d)


def test_chaining_is_exact():
    """P7: running T1 tokens, then T2 tokens from the carried state, gives the
    same outputs and final state as one run over T1 + T2 tokens."""
    rng = np.random.default_rng(16)
    B, T, H, d = 1, 50, 2, 32
    q, k, v, g, beta, h0 = _rand_case(rng, B, T, H, d, d)
    o, hT = oracle.forward(q, k, v, g, beta, 0.2, h0, threads=2)
    s = 23
    oa, ha = oracle.forward(q[:, :s], k[:, :s], v[:, :s], g[:, :s], beta[:, :s], 0.2, h0)
    ob, hb = oracle.forward(q[:, s:], k[:, s:], v[:, s:], g[:, s:], beta[:, s:], 0.2, ha)
    np.testing.assert_array_equal(np.concatenate([oa, ob], axis=1), o)
    np.testing.assert_array_equal(hb, hT)


def test_norm_invariance():
    """P9: q and k are L2-normalised inside the operation, so positive scalings
    of them (per token) change nothing (exactly so at eps = 0)."""
    rng = np.random.default_rng(17)
    B, T, H, d = 1, 30, 2, 16
    q, k, v, g, beta, h0 = _rand_case(rng, B, T, H, d, d)
    cq = rng.uniform(0.1, 10.0, (B, T, H, 1))
    ck = rng.uniform(0.1, 10.0, (B, T, H, 1))
    o, hT = oracle.forward(q, k, v, g, beta, 1.0, h0, eps=0.0, threads=1)
    o2, hT2 = oracle.forward(q * cq, k * ck, v, g, beta, 1.0, h0, eps=0.0, threads=1)
    assert _rel(o2, o) < 1e-13 and _rel(hT2, hT) < 1e-13


def test_linearity_in_values_and_state():
    """P10: for fixed q, k, g, beta the map (V, h0) -> (O, hT) is linear, and
    value column j only ever touches column j."""
    rng = np.random.default_rng(18)
    B, T, H, d = 1, 40, 1, 16
    q, k, v1, g, beta, h1 = _rand_case(rng, B, T, H, d, d)
    v2 = rng.standard_normal(v1.shape)
    h2 = rng.standard_normal(h1.shape)
    a, b = 0.7, -1.3
    o1, s1 = oracle.forward(q, k, v1, g, beta, 1.0, h1, threads=1)
    o2, s2 = oracle.forward(q, k, v2, g, beta, 1.0, h2, threads=1)
    o3, s3 = oracle.forward(q, k, a * v1 + b * v2, g, beta, 1.0, a * h1 + b * h2, threads=1)
    assert _rel(o3, a * o1 + b * o2) < 1e-12 and _rel(s3, a * s1 + b * s2) < 1e-12
    v4 = v1.copy()
    v4[..., 5] += 1.0
    o4, s4 = oracle.forward(q, k, v4, g, beta, 1.0, h1, threads=1)
    cols = np.arange(d) != 5
    np.testing.assert_array_equal(o4[..., cols], o1[..., cols])
    np.testing.assert_array_equal(s4[..., cols], s1[..., cols])
    assert np.abs(o4[..., 5] - o1[..., 5]).max() > 1e-3


def test_contractive_transition():
    """P14: for g <= 0, beta in [0, 2] and a unit key, the per-token
    transition (I - beta kh kh^T) Diag(exp g) has spectral norm <= 1, so the
    state grows by at most beta |v| per token and errors do not amplify."""
    rng = np.random.default_rng(19)
    d = 32
    for _ in range(50):
        k = rng.standard_normal((1, d))
        g = -rng.uniform(0, 5, (1, d))
        beta = rng.uniform(0, 2, 1)
        Ms, _ = tp.transition_matrices(k, g, beta, eps=0.0)
        assert np.linalg.norm(Ms[0], 2) <= 1.0 + 1e-12
    q, k, v, g, beta, h0 = _rand_case(rng, 1, 1, 1, d, d)
    _, hT = oracle.forward(q, k, v, g, beta, 1.0, h0, eps=0.0, threads=1)
    bound = np.linalg.norm(h0[0, 0], 2) + beta[0, 0, 0] * np.linalg.norm(v[0, 0, 0])
    assert np.linalg.norm(hT[0, 0], 2) <= bound + 1e-12


def test_decode_step_matches_forward():
    """One decode step is one token of the recurrence applied to S."""
    rng = np.random.default_rng(20)
    B, H, d = 3, 2, 16
    q, k, v, g, beta, S = _rand_case(rng, B, 1, H, d, d)
    o, hT = oracle.forward(q, k, v, g, beta, 0.9, S, threads=1)
    o1, S1 = oracle.step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], 0.9, S, threads=1)
    np.testing.assert_array_equal(o1, o[:, 0])
    np.testing.assert_array_equal(S1, hT)


# ---------------------------------------------------------------------------
# short convolution + SiLU in front of the attention
# ---------------------------------------------------------------------------
def test_silu_textbook_values():
    """With the current-token tap 1 and the others 0 the filter is the
    identity, so the output is SiLU of the input: x * logistic(x), checked
    against logistic values written out (1/(1+e) and friends)."""
    xs = np.array([0.0, 1.0, -1.0, 2.0, -3.0])
    # x / (1 + e^-x): 0, 0.7310585786300049, -0.2689414213699951,
    # 1.7615941559557649, -0.14227761953270035
    want = np.array([0.0, 0.7310585786300049, -0.2689414213699951, 1.7615941559557649,
                     -0.14227761953270035])
    x = xs.reshape(1, -1, 1, 1)
    w = np.zeros((1, 1, 4))
    w[0, 0, 3] = 1.0
    y, _ = oracle.short_conv_silu(x, w)
    np.testing.assert_allclose(y.reshape(-1), want, rtol=1e-15, atol=1e-16)


def test_short_conv_impulse_response():
    """An impulse a at token t0 reaches token t0 + m (m = 0..3) through tap
    3 - m: the output there is SiLU(w[3 - m] a) and zero everywhere else.
    This fixes the tap order (tap 3 = current token, tap 0 = three back)."""
    T, t0, a = 10, 4, 1.5
    w = np.array([0.3, -0.7, 1.1, 0.5]).reshape(1, 1, 4)
    x = np.zeros((1, T, 1, 1))
    x[0, t0, 0, 0] = a
    y, _ = oracle.short_conv_silu(x, w)
    want = np.zeros(T)
    for m in range(4):
        z = w[0, 0, 3 - m] * a
        want[t0 + m] = z / (1.0 + math.exp(-z))
    np.testing.assert_allclose(y.reshape(-1), want, rtol=1e-15, atol=1e-17)


def test_short_conv_state_and_split():
    """Causal with a 3-token state: filtering x[:t1] and then x[t1:] from the
    state the first call returns equals filtering x whole, for every split;
    and the first output of a zero input reads only the state."""
    rng = np.random.default_rng(7)
    B, T, H, D = 2, 11, 3, 5
    x = rng.standard_normal((B, T, H, D))
    w = rng.standard_normal((H, D, 4))
    s0 = rng.standard_normal((B, 3, H, D))
    whole, s_end = oracle.short_conv_silu(x, w, s0)
    for t1 in range(0, T + 1):
        y1, s1 = oracle.short_conv_silu(x[:, :t1], w, s0)
        y2, s2 = oracle.short_conv_silu(x[:, t1:], w, s1)
        np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), whole, rtol=0, atol=0)
        np.testing.assert_array_equal(s2, s_end)
    np.testing.assert_array_equal(s_end, x[:, T - 3:])
    y, _ = oracle.short_conv_silu(np.zeros((B, 1, H, D)), w, s0)
    pre = w[None, :, :, 0] * s0[:, 0] + w[None, :, :, 1] * s0[:, 1] + w[None, :, :, 2] * s0[:, 2]
    np.testing.assert_allclose(y[:, 0], pre / (1.0 + np.exp(-pre)), rtol=1e-14, atol=1e-15)


def test_decode_conv_steps_match_forward_conv():
    """Decoding token by token with the carried conv state and attention
    state reproduces the prefill over the same tokens: step_conv is the
    filter of one new token plus one step, and both agree with forward_conv
    (whose filter and recurrence are pinned above) at every token."""
    rng = np.random.default_rng(11)
    B, T, H, D = 2, 6, 3, 8
    q, k, v = (rng.standard_normal((B, T, H, D)) for _ in range(3))
    wq, wk, wv = (rng.standard_normal((H, D, 4)) for _ in range(3))
    g = -5.0 / (1.0 + np.exp(-(rng.standard_normal((B, T, H, D)) - 1.0)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = 0.1 * rng.standard_normal((B, H, D, D))
    cs0 = tuple(rng.standard_normal((B, 3, H, D)) for _ in range(3))
    o, hT, cs_end = oracle.forward_conv(q, k, v, wq, wk, wv, g, beta, 0.7, S0, cs0, threads=1)
    S, cs = S0.copy(), cs0
    for t in range(T):
        ot, S, cs = oracle.step_conv(q[:, t], k[:, t], v[:, t], wq, wk, wv, cs, g[:, t],
                                     beta[:, t], 0.7, S, threads=1)
        np.testing.assert_allclose(ot, o[:, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, hT, rtol=1e-12, atol=1e-13)
    for a, b in zip(cs, cs_end):
        np.testing.assert_array_equal(a, b)


def test_round_bf16_matches_torch_conversion():
    """round_bf16 equals torch's fp32 -> bfloat16 conversion (round to
    nearest, ties to even) on random values, on exact ties in both
    directions, and below the fp32 -> bf16 rounding of fp64 inputs."""
    import torch
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, -2.5, 3.0e38, 1e-40]])
    # ties: bf16 value plus half an ulp, with an even and an odd last bit
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8),
                     -(1.0 + 3 * 2.0 ** -8)])
    x = np.concatenate([x, ties])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.round_bf16(x), want)
    np.testing.assert_array_equal(oracle.round_bf16(ties), [1.0, 1.0 + 2.0 ** -6, -1.0,
                                                           -(1.0 + 2.0 ** -6)])


def test_short_conv_rounded_output_is_the_bf16_of_the_exact_output():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 9, 2, 4))
    w = rng.standard_normal((2, 4, 4))
    y, _ = oracle.short_conv_silu(x, w)
    yr, _ = oracle.short_conv_silu(x, w, round_out=True)
    np.testing.assert_array_equal(yr, oracle.round_bf16(y))
    assert np.abs(yr - y).max() <= 2.0 ** -8 * np.abs(y).max()  # half an ulp of 8 bits


def test_output_gate_values():
    """The gate is the logistic function of its logit: at 0 it halves the
    output exactly, at a large logit it passes it (1 / (1 + e^-40) rounds to
    1 in fp64), and at +-1, 2, -3 it takes the logistic values written out
    (the SiLU pin's values divided by x)."""
    o = np.array([[2.0, -3.0, 5.0, 7.0, 1.0, -1.0]])
    z = np.array([[0.0, 0.0, 40.0, 1.0, -1.0, 2.0]])
    want = np.array([[1.0, -1.5, 5.0, 7.0 * 0.7310585786300049, 0.2689414213699951,
                      -0.8807970779778823]])
    np.testing.assert_allclose(oracle.output_gate(o, z), want, rtol=1e-15, atol=0)
    np.testing.assert_allclose(oracle.output_gate(np.array([3.0]), np.array([-3.0])),
                               [3.0 * 0.04742587317756678], rtol=1e-14)


def test_gated_conv_forward_and_steps():
    """forward_conv with a gate equals the ungated output times the gate's
    logistic; with zero logits exactly half; and step_conv with the same
    gate per token reproduces it."""
    rng = np.random.default_rng(13)
    B, T, H, D = 1, 5, 2, 8
    q, k, v = (rng.standard_normal((B, T, H, D)) for _ in range(3))
    wq, wk, wv = (rng.standard_normal((H, D, 4)) for _ in range(3))
    g = -5.0 / (1.0 + np.exp(-(rng.standard_normal((B, T, H, D)) - 1.0)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    z = rng.standard_normal((B, T, H, D))
    o, hT, _ = oracle.forward_conv(q, k, v, wq, wk, wv, g, beta, 0.7, threads=1)
    og, hg, _ = oracle.forward_conv(q, k, v, wq, wk, wv, g, beta, 0.7, threads=1, gate=z)
    oh, _, _ = oracle.forward_conv(q, k, v, wq, wk, wv, g, beta, 0.7, threads=1,
                                   gate=np.zeros_like(z))
    np.testing.assert_array_equal(hg, hT)
    np.testing.assert_array_equal(oh, 0.5 * o)
    np.testing.assert_allclose(og, o / (1.0 + np.exp(-z)), rtol=1e-15)
    S = np.zeros((B, H, D, D))
    cs = tuple(np.zeros((B, 3, H, D)) for _ in range(3))
    for t in range(T):
        ot, S, cs = oracle.step_conv(q[:, t], k[:, t], v[:, t], wq, wk, wv, cs, g[:, t],
                                     beta[:, t], 0.7, S, threads=1, gate=z[:, t])
        np.testing.assert_allclose(ot, og[:, t], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# backward of one recurrent step
# ---------------------------------------------------------------------------
def _step_loss(x, d_o, dS_next, scale):
    o, Sn = oracle.step(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, x["S"], threads=1)
    return float(np.sum(d_o * o) + np.sum(dS_next * Sn))


def test_step_backward_against_finite_differences():
    """Every gradient of one step (q, k, v, g, beta and the previous state)
    against central differences of the forward step in fp64: a dropped term,
    a wrong sign or a transposed operand anywhere in the reverse pass fails
    here.  Small D so that every entry is perturbed."""
    rng = np.random.default_rng(21)
    B, H, D, scale = 1, 2, 6, 0.8
    x = {"q": rng.standard_normal((B, H, D)), "k": rng.standard_normal((B, H, D)),
         "v": rng.standard_normal((B, H, D)),
         "g": -5.0 / (1.0 + np.exp(-rng.standard_normal((B, H, D)))),
         "beta": 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H)))),
         "S": rng.standard_normal((B, H, D, D))}
    d_o = rng.standard_normal((B, H, D))
    dS_next = rng.standard_normal((B, H, D, D))
    grads = oracle.step_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, x["S"],
                                 d_o, dS_next)
    h = 1e-6
    for name, gr in zip(("q", "k", "v", "g", "beta", "S"), grads):
        num = np.zeros_like(x[name])
        for idx in np.ndindex(*x[name].shape):
            xp = {k_: v_.copy() for k_, v_ in x.items()}
            xm = {k_: v_.copy() for k_, v_ in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            num[idx] = (_step_loss(xp, d_o, dS_next, scale) -
                        _step_loss(xm, d_o, dS_next, scale)) / (2 * h)
        np.testing.assert_allclose(gr, num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_step_backward_chains_to_the_sequence_gradient():
    """Backpropagating token by token through stored states gives the
    gradient of the whole T-token forward pass (checked by central
    differences of forward), including that of the initial state."""
    rng = np.random.default_rng(22)
    B, T, H, D, scale = 1, 4, 1, 5, 0.9
    q, k, v = (rng.standard_normal((B, T, H, D)) for _ in range(3))
    g = -5.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, D))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    h0 = rng.standard_normal((B, H, D, D))
    d_o = rng.standard_normal((B, T, H, D))
    d_hT = rng.standard_normal((B, H, D, D))

    def loss(h0_, v_):
        o, hT = oracle.forward(q, k, v_, g, beta, scale, h0_, threads=1)
        return float(np.sum(d_o * o) + np.sum(d_hT * hT))

    states = [h0]
    for t in range(T):
        _, Sn = oracle.step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], scale, states[-1],
                            threads=1)
        states.append(Sn)
    dS = d_hT.copy()
    dv = np.zeros_like(v)
    for t in reversed(range(T)):
        _, _, dv_t, _, _, dS = oracle.step_backward(q[:, t], k[:, t], v[:, t], g[:, t],
                                                    beta[:, t], scale, states[t], d_o[:, t], dS)
        dv[:, t] = dv_t
    eps = 1e-6
    num_h0 = np.zeros_like(h0)
    for idx in np.ndindex(*h0.shape):
        hp, hm = h0.copy(), h0.copy()
        hp[idx] += eps
        hm[idx] -= eps
        num_h0[idx] = (loss(hp, v) - loss(hm, v)) / (2 * eps)
    np.testing.assert_allclose(dS, num_h0, rtol=1e-6, atol=1e-7)
    num_v = np.zeros_like(v)
    for idx in np.ndindex(*v.shape):
        vp, vm = v.copy(), v.copy()
        vp[idx] += eps
        vm[idx] -= eps
        num_v[idx] = (loss(h0, vp) - loss(h0, vm)) / (2 * eps)
    np.testing.assert_allclose(dv, num_v, rtol=1e-6, atol=1e-7)


def _chained_step_backward(q, k, v, g, beta, scale, h0, d_o, d_hT):
    """Reference: step_backward chained over the kept states (itself pinned
    to central differences above)."""
    B, T, H, D = q.shape
    states = [h0]
    for t in range(T):
        _, Sn = oracle.step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], scale, states[-1],
                            threads=1)
        states.append(Sn)
    dS = d_hT.copy()
    out = [np.zeros_like(x) for x in (q, k, v, g)] + [np.zeros_like(beta)]
    for t in reversed(range(T)):
        r = oracle.step_backward(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], scale,
                                 states[t], d_o[:, t], dS)
        for j in range(4):
            out[j][:, t] = r[j]
        out[4][:, t] = r[4]
        dS = r[5]
    return (*out, dS)


@pytest.mark.parametrize("chunk", [4, 16, 64])
def test_chunk_backward_equals_chained_steps(chunk):
    """The chunkwise backward (chunk algebra, differentiated in reverse) gives
    the gradients of the token-by-token chain for every chunk size, with a
    partial last chunk, decays down to the -5 bound and a nonzero initial
    state: a wrong term in the chunk form's derivative fails here."""
    rng = np.random.default_rng(31)
    B, T, H, D, scale = 1, 37, 2, 6, 0.8
    q, k, v = (rng.standard_normal((B, T, H, D)) for _ in range(3))
    g = -5.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, D)) * 2.0))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    h0 = 0.3 * rng.standard_normal((B, H, D, D))
    d_o = rng.standard_normal((B, T, H, D))
    d_hT = rng.standard_normal((B, H, D, D))
    got = oracle.chunk_backward(q, k, v, g, beta, scale, h0, d_o, d_hT, chunk=chunk)
    want = _chained_step_backward(q, k, v, g, beta, scale, h0, d_o, d_hT)
    for name, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got, want):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-11, err_msg=name)


# ---------------------------------------------------------------------------
# backward of the whole recurrence, token by token (the reference of every GPU
# backward comparison)
# ---------------------------------------------------------------------------
def test_sequence_backward_against_finite_differences():
    """Every gradient of the T-token forward (q, k, v, g, beta, the initial
    state) against central differences of ``forward`` itself, in fp64, with a
    final-state gradient and decays down to the -5 bound: a dropped term, a
    wrong sign, a token off by one or a transposed operand in the C reverse
    pass fails here.  Two sequences (B = 1, H = 2) so the sequence indexing of
    the layout is exercised too."""
    rng = np.random.default_rng(41)
    B, T, H, D, scale = 1, 9, 2, 5, 0.85
    x = {"q": rng.standard_normal((B, T, H, D)), "k": rng.standard_normal((B, T, H, D)),
         "v": rng.standard_normal((B, T, H, D)),
         "g": -5.0 / (1.0 + np.exp(-2.0 * rng.standard_normal((B, T, H, D)))),
         "beta": 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H)))),
         "h0": rng.standard_normal((B, H, D, D))}
    d_o = rng.standard_normal((B, T, H, D))
    d_hT = rng.standard_normal((B, H, D, D))

    def loss(y):
        o, hT = oracle.forward(y["q"], y["k"], y["v"], y["g"], y["beta"], scale, y["h0"],
                               threads=1)
        return float(np.sum(d_o * o) + np.sum(d_hT * hT))

    grads = oracle.sequence_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], scale,
                                     x["h0"], d_o, d_hT, threads=2)
    h = 1e-6
    for name, gr in zip(("q", "k", "v", "g", "beta", "h0"), grads):
        assert gr.shape == x[name].shape, name
        num = np.zeros_like(x[name])
        for idx in np.ndindex(*x[name].shape):
            xp = {k_: v_.copy() for k_, v_ in x.items()}
            xm = {k_: v_.copy() for k_, v_ in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            num[idx] = (loss(xp) - loss(xm)) / (2 * h)
        np.testing.assert_allclose(gr, num, rtol=2e-6, atol=2e-7, err_msg=name)


def test_sequence_backward_equals_chained_step_backward():
    """The C sequence backward is the chain of the (separately pinned) Python
    step backward over the kept states, to rounding, with B = 2 and zero or
    absent initial state and final gradient."""
    rng = np.random.default_rng(42)
    B, T, H, D, scale = 2, 23, 3, 7, 0.6
    q, k, v = (rng.standard_normal((B, T, H, D)) for _ in range(3))
    g = -5.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, D))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    d_o = rng.standard_normal((B, T, H, D))
    for h0, d_hT in ((0.3 * rng.standard_normal((B, H, D, D)), rng.standard_normal((B, H, D, D))),
                     (None, None)):
        got = oracle.sequence_backward(q, k, v, g, beta, scale, h0, d_o, d_hT, threads=3)
        z = np.zeros((B, H, D, D))
        want = _chained_step_backward(q, k, v, g, beta, scale, z if h0 is None else h0, d_o,
                                      z if d_hT is None else d_hT)
        for name, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got, want):
            np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12, err_msg=name)


def test_sequence_backward_empty_sequence():
    """No tokens: the final-state gradient passes through to the initial one."""
    rng = np.random.default_rng(43)
    B, H, D = 2, 2, 4
    e = np.zeros((B, 0, H, D))
    d_hT = rng.standard_normal((B, H, D, D))
    r = oracle.sequence_backward(e, e, e, e, np.zeros((B, 0, H)), 1.0, None, e, d_hT)
    np.testing.assert_array_equal(r[5], d_hT)
    assert r[0].shape == (B, 0, H, D) and r[4].shape == (B, 0, H)
