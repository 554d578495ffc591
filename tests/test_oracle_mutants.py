"""The oracle's pins reject plausible mistakes in the oracle itself.

Each case plants one mistake in a copy of oracle/kda_oracle.c (a dropped term
or factor, a wrong sign, a wrong operand, an off-by-one token, two steps in
the wrong order), builds the copy with gcc and runs the pins of
test_oracle_pins.py against it: at least one of them must fail.  The same is
done for the Python side of the oracle (oracle/oracle.py: the short
convolution, SiLU, the bf16 rounding, the output gate and the one-step
backward), whose mutated copy is loaded as a module of its own.  The copy
without a mistake passes all of them, so every failure comes from the planted
mistake.  The forward mistakes follow the recurrence of the Kimi-K3 深度解析
blog, section 三 (per-channel decay, prediction from the decayed state, the
error beta (v - prediction) written along the key) with the in-kernel L2
normalisation of the 深入 Kimi-K3 thread's KDA paragraph; the backward ones
its reverse-mode derivative.  Everything here runs on the CPU.
"""
import ctypes
import os
import subprocess
import types

import pytest

import test_oracle_pins as pins
from oracle import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")


def _nth(src, old, new, n=0):
    """src with occurrence n of old replaced by new (the text must be there)."""
    at = -1
    for _ in range(n + 1):
        at = src.find(old, at + 1)
        assert at >= 0, f"mutation site not found: {old!r} (occurrence {n})"
    return src[:at] + new + src[at + len(old):]


def _swap_blocks(src, first, second, end):
    """src with the block starting at marker `first` and the one starting at
    `second` (which ends at marker `end`) exchanged; the markers are comment
    lines of the forward loop."""
    a = src.index(first)
    b = src.index(second, a)
    c = src.index(end, b)
    return src[:a] + src[b:c] + src[a:b] + src[c:]


DECAY = "        /* decay: every key row i is scaled by exp(g_t[i]) */"
PRED = "        /* prediction p = S^T kh from the decayed state */"
ERR = "        /* error term u = beta (v - p) */"
WRITE = "        /* delta-rule write S += kh u^T */"
READ = "        /* read-out o = scale S^T qh, after the write */"
READ_END = "    if (jb->hT) memcpy(jb->hT"

# name -> function of the source text.  "forward" cases change the recurrence
# (run_sequence), "backward" cases its derivative (backward_sequence; its own
# replay of the forward is left alone unless named).
MUTANTS = {
    # forward
    "fwd: no decay": lambda s: _nth(s, "row[j] *= a;", "row[j] *= 1.0;"),
    "fwd: decay with the sign of g flipped": lambda s: _nth(
        s, "const double a = exp(gt[i]);", "const double a = exp(-gt[i]);"),
    "fwd: error with + p": lambda s: _nth(
        s, "u[j] = beta[t] * (vt[j] - p[j]);", "u[j] = beta[t] * (vt[j] + p[j]);"),
    "fwd: beta dropped": lambda s: _nth(
        s, "u[j] = beta[t] * (vt[j] - p[j]);", "u[j] = (vt[j] - p[j]);"),
    "fwd: prediction from the undecayed state": lambda s: _swap_blocks(s, DECAY, PRED, ERR),
    "fwd: read-out before the write": lambda s: _swap_blocks(s, WRITE, READ, READ_END),
    "fwd: read-out with the key": lambda s: _nth(
        s, "ot[j] += qh[i] * row[j];", "ot[j] += kh[i] * row[j];"),
    "fwd: write along the query": lambda s: _nth(
        s, "for (int j = 0; j < dv; ++j) row[j] += kh[i] * u[j];",
        "for (int j = 0; j < dv; ++j) row[j] += qh[i] * u[j];"),
    "fwd: k not normalised": lambda s: _nth(
        s, "kh[i] = nk > 0.0 ? kt[i] / nk : 0.0;", "kh[i] = kt[i];"),
    "fwd: q not normalised": lambda s: _nth(
        s, "qh[i] = nq > 0.0 ? qt[i] / nq : 0.0;", "qh[i] = qt[i];"),
    "fwd: eps left out of the norms": lambda s: _nth(
        s, "const double nq = sqrt(sq + jb->eps), nk = sqrt(sk + jb->eps);",
        "const double nq = sqrt(sq), nk = sqrt(sk);"),
    "fwd: scale dropped": lambda s: _nth(s, "ot[j] *= jb->scale;", "ot[j] *= 1.0;"),
    "fwd: h0 ignored": lambda s: _nth(
        s, "if (jb->h0)\n        memcpy(S, jb->h0", "if (0)\n        memcpy(S, jb->h0"),
    "fwd: prediction from the transposed state": lambda s: _nth(
        s, "for (int j = 0; j < dv; ++j) p[j] += kh[i] * row[j];",
        "for (int j = 0; j < dv; ++j) p[j] += kh[i] * S[((size_t)j * dk + i) % ((size_t)dk * dv)];"),
    "fwd: decay of the token before": lambda s: _nth(
        s, "const double *vt = v + (size_t)t * dv, *gt = g + (size_t)t * dk;",
        "const double *vt = v + (size_t)t * dv, *gt = g + (size_t)(t > 0 ? t - 1 : 0) * dk;"),
    # backward
    "bwd: dp with the wrong sign": lambda s: _nth(s, "dp[j] = -bt * du[j];", "dp[j] = bt * du[j];"),
    "bwd: dbeta without the prediction": lambda s: _nth(
        s, "db += du[j] * (vt[j] - p[j]);", "db += du[j] * vt[j];"),
    "bwd: state gradient not decayed back": lambda s: _nth(
        s, "G[(size_t)i * dv + j] = a[i] * dst;", "G[(size_t)i * dv + j] = dst;"),
    "bwd: dg from the state before the decay": lambda s: _nth(
        s, "dgi += St[(size_t)i * dv + j] * dst;", "dgi += Sp[(size_t)i * dv + j] * dst;"),
    "bwd: dq without the norm's projection": lambda s: _nth(
        s, "(dqh[i] - qh[i] * qd) / nq", "dqh[i] / nq"),
    "bwd: dk without the norm's projection": lambda s: _nth(
        s, "(dkh[i] - kh[i] * kd) / nk", "dkh[i] / nk"),
    "bwd: scale dropped from dq": lambda s: _nth(s, "dqh[i] = jb->scale * acc;", "dqh[i] = acc;"),
    "bwd: dk misses the prediction's term": lambda s: _nth(s, "dkh[i] += acc;", "dkh[i] += 0.0 * acc;"),
    "bwd: read-out gradient not carried into the state": lambda s: _nth(
        s, "G[(size_t)i * dv + j] += jb->scale * qh[i] * dot[j];",
        "G[(size_t)i * dv + j] += 0.0 * qh[i] * dot[j];"),
    "bwd: dv without beta": lambda s: _nth(
        s, "jb->dvv[((size_t)s * T + t) * dv + j] = bt * du[j];",
        "jb->dvv[((size_t)s * T + t) * dv + j] = du[j];"),
    "bwd: d_hT ignored": lambda s: _nth(
        s, "if (jb->d_hT)\n        memcpy(G", "if (0)\n        memcpy(G"),
}

# The pins of the oracle, each a callable that raises when its fact fails.
PINS = {
    "golden hand example": pins.test_golden_hand_example,
    "transition product 4x3": lambda: pins.test_transition_product(4, 3, 1),
    "transition product 8x8": lambda: pins.test_transition_product(8, 8, 5),
    "transition product 16x12": lambda: pins.test_transition_product(16, 12, 8),
    "orthonormal recall, basis": lambda: pins.test_orthonormal_recall("basis"),
    "orthonormal recall, hadamard": lambda: pins.test_orthonormal_recall("hadamard"),
    "beta=1 recall, random g": lambda: pins.test_beta_one_exact_recall("random"),
    "beta=1 recall, g at the bound": lambda: pins.test_beta_one_exact_recall("bound"),
    "beta=1 recall, g=0": lambda: pins.test_beta_one_exact_recall("zero"),
    "beta=0 pure decay": pins.test_beta_zero_pure_decay,
    "read only": pins.test_read_only,
    "chaining": pins.test_chaining_is_exact,
    "norm invariance": pins.test_norm_invariance,
    "linearity": pins.test_linearity_in_values_and_state,
    "contraction": pins.test_contractive_transition,
    "backward vs finite differences": pins.test_sequence_backward_against_finite_differences,
    "backward vs chained step backward": pins.test_sequence_backward_equals_chained_step_backward,
    "backward of an empty sequence": pins.test_sequence_backward_empty_sequence,
}


def _build(src_text, tmp_path, name):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src_text)
    subprocess.run(["gcc", "-O2", "-std=c99", "-shared", "-fPIC", "-pthread", str(c), "-o",
                    str(so), "-lm"], check=True, capture_output=True)
    return oracle.configure(ctypes.CDLL(str(so)))


def _failing_pins(lib, monkeypatch):
    monkeypatch.setattr(oracle, "_lib", lib)
    failed = []
    for name, pin in PINS.items():
        try:
            pin()
        except Exception:  # an assertion, or a numerical error from the mistake
            failed.append(name)
    return failed


def test_pins_pass_on_an_unmodified_copy(tmp_path, monkeypatch):
    with open(SRC) as f:
        src = f.read()
    assert _failing_pins(_build(src, tmp_path, "copy"), monkeypatch) == []


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_pins_reject_a_planted_mistake(mutant, tmp_path, monkeypatch):
    with open(SRC) as f:
        src = f.read()
    bad = MUTANTS[mutant](src)
    assert bad != src
    failed = _failing_pins(_build(bad, tmp_path, "mutant"), monkeypatch)
    print(f"{mutant}: caught by {failed}")
    assert failed, f"no pin rejects the mistake '{mutant}'"


# Mistakes in oracle/oracle.py (the same kinds), each against the pins that
# use that part.
PY_MUTANTS = {
    "silu with the logistic of -x": lambda s: _nth(
        s, "return x / (1.0 + np.exp(-x))", "return x / (1.0 + np.exp(x))"),
    "bf16 rounding by truncation": lambda s: _nth(
        s, "r = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)",
        "r = bits & np.uint32(0xFFFF0000)"),
    "bf16 rounding with ties down": lambda s: _nth(
        s, "r = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)",
        "r = (bits + np.uint32(0x7FFF)) & np.uint32(0xFFFF0000)"),
    "conv taps in reverse order": lambda s: _nth(
        s, "pre += w[None, None, :, :, j] * full[:, j:j + T]",
        "pre += w[None, None, :, :, CONV_TAPS - 1 - j] * full[:, j:j + T]"),
    "conv state ignored": lambda s: _nth(
        s, "prev = np.zeros((B, CONV_TAPS - 1, H, D)) if state is None else _f64(state)",
        "prev = np.zeros((B, CONV_TAPS - 1, H, D))"),
    "conv state returned one token early": lambda s: _nth(
        s, "np.ascontiguousarray(full[:, T:])", "np.ascontiguousarray(full[:, T - 1:T + 2])"),
    "gate with the logistic of -z": lambda s: _nth(
        s, "return _f64(o) / (1.0 + np.exp(-_f64(z)))", "return _f64(o) / (1.0 + np.exp(_f64(z)))"),
    "step backward: dp with the wrong sign": lambda s: _nth(s, "dp = -bt * du", "dp = bt * du"),
    "step backward: state gradient not decayed back": lambda s: _nth(
        s, "dS_prev[b, h] = a[:, None] * dSt", "dS_prev[b, h] = dSt"),
    "step backward: dg from the state before the decay": lambda s: _nth(
        s, "dg[b, h] = np.sum(St * dSt, axis=1)", "dg[b, h] = np.sum(S_prev[b, h] * dSt, axis=1)"),
    "step backward: dq without the norm's projection": lambda s: _nth(
        s, "dq[b, h] = rq * dqh - rq ** 3 * (q[b, h] @ dqh) * q[b, h]", "dq[b, h] = rq * dqh"),
    "step backward: dk misses the prediction's term": lambda s: _nth(
        s, "dkh += St @ dp", "dkh += 0.0 * (St @ dp)"),
    "step backward: read-out gradient without the scale": lambda s: _nth(
        s, "G = dS_next[b, h] + scale * np.outer(qh, d_o[b, h])",
        "G = dS_next[b, h] + np.outer(qh, d_o[b, h])"),
}

PY_PINS = {
    "silu values": pins.test_silu_textbook_values,
    "conv impulse response": pins.test_short_conv_impulse_response,
    "conv state and split": pins.test_short_conv_state_and_split,
    "decode conv steps": pins.test_decode_conv_steps_match_forward_conv,
    "bf16 rounding vs torch": pins.test_round_bf16_matches_torch_conversion,
    "rounded conv output": pins.test_short_conv_rounded_output_is_the_bf16_of_the_exact_output,
    "gate values": pins.test_output_gate_values,
    "gated conv": pins.test_gated_conv_forward_and_steps,
    "step backward vs finite differences": pins.test_step_backward_against_finite_differences,
    "step backward chained vs sequence gradient": pins.test_step_backward_chains_to_the_sequence_gradient,
    "sequence backward vs chained step backward": pins.test_sequence_backward_equals_chained_step_backward,
}


def _py_module(src_text):
    """The oracle module built from src_text; it loads the same C library."""
    mod = types.ModuleType("oracle_copy")
    mod.__file__ = oracle.__file__
    exec(compile(src_text, oracle.__file__, "exec"), mod.__dict__)
    return mod


def _failing_py_pins(mod, monkeypatch):
    monkeypatch.setattr(pins, "oracle", mod)
    failed = []
    for name, pin in PY_PINS.items():
        try:
            pin()
        except Exception:  # an assertion, or a numerical error from the mistake
            failed.append(name)
    return failed


def test_python_pins_pass_on_an_unmodified_copy(monkeypatch):
    with open(oracle.__file__) as f:
        src = f.read()
    assert _failing_py_pins(_py_module(src), monkeypatch) == []


@pytest.mark.parametrize("mutant", list(PY_MUTANTS))
def test_python_pins_reject_a_planted_mistake(mutant, monkeypatch):
    with open(oracle.__file__) as f:
        src = f.read()
    bad = PY_MUTANTS[mutant](src)
    assert bad != src
    failed = _failing_py_pins(_py_module(bad), monkeypatch)
    print(f"{mutant}: caught by {failed}")
    assert failed, f"no pin rejects the mistake '{mutant}'"
