"""GPU parity of kda_recurrent_step_bwd_f32 (backward of one fp32 recurrent
step) against the fp64 oracle's step_backward, which is pinned by central
differences of the forward step; and backpropagation through a short
sequence with the states kept, against the oracle chained the same way.

fp32 arithmetic throughout: with fp32 I/O the bar is the fp32-mode one, 1e-3
normalised max error per gradient (the measured errors are near 1e-6); with
bf16 q / k / v / dout the oracle reads the same bf16 values and dq, dk, dv
are rounded to bf16, so the bar is the bf16 one, 1e-2."""
import numpy as np
import pytest
import torch

from kda_check import host64, say
from linear_attention_07_amd import libkda, synth
from oracle import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-3
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS_prev")


def rel(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(x - ref).max() / (den if den > 0 else 1.0))


def inputs(B, H, seed, io=torch.float32):
    x = synth.decode_step_inputs(B, H, io, seed=seed, step=0, device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(seed)
    x["S"] = 0.1 * torch.randn((B, H, 128, 128), generator=gen, device=DEV)
    x["dout"] = torch.randn((B, H, 128), generator=gen, device=DEV).to(io)
    x["dS"] = 0.1 * torch.randn((B, H, 128, 128), generator=gen, device=DEV)
    return x


def gpu_bwd(x):
    dS = x["dS"].clone()
    grads = libkda.recurrent_step_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"],
                                      x["S"], x["dout"], dS)
    torch.cuda.synchronize()
    return (*grads, dS)


def oracle_bwd(x, sel=slice(None)):
    h = lambda t: host64(t[sel])
    return oracle.step_backward(h(x["q"]), h(x["k"]), h(x["v"]), h(x["g"]), h(x["beta"]),
                                x["scale"], h(x["S"]), h(x["dout"]), h(x["dS"]))


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,H", [(1, 1), (3, 5), (2, 8)])
def test_step_bwd_against_oracle(B, H, io):
    x = inputs(B, H, seed=800 + 10 * B + H, io=io)
    got = gpu_bwd(x)
    want = oracle_bwd(x)
    errs = {n: rel(host64(a), b) for n, a, b in zip(NAMES, got, want)}
    say(f"step bwd B={B} H={H} {io}: " + " ".join(f"{n} {e:.1e}" for n, e in errs.items()))
    assert max(errs.values()) <= (TOL if io == torch.float32 else 1e-2)
    if io == torch.bfloat16:   # the fp32 outputs keep fp32 accuracy
        assert max(errs["dg"], errs["dbeta"], errs["dS_prev"]) <= TOL


def test_step_bwd_b256_sampled():
    """The batched decode shape (B = 256, H = 96): every gradient of 64
    sampled sequences against the oracle."""
    B, H = 256, 96
    x = inputs(B, H, seed=811)
    got = gpu_bwd(x)
    bs = list(range(0, B, 4))
    want = oracle_bwd(x, sel=bs)
    errs = {n: rel(host64(a[bs]), b) for n, a, b in zip(NAMES, got, want)}
    say("step bwd b256 (64 sequences): " + " ".join(f"{n} {e:.1e}" for n, e in errs.items()))
    assert max(errs.values()) <= TOL


def test_bptt_through_a_sequence():
    """Forward T steps with kda_recurrent_step_f32 keeping every state, then
    T backward steps in reverse: the gradients of every token's inputs and of
    the initial state match the oracle chained through the same states."""
    B, H, T = 2, 3, 24
    gen = torch.Generator(device=DEV).manual_seed(820)
    S0 = 0.1 * torch.randn((B, H, 128, 128), generator=gen, device=DEV)
    xs = [synth.decode_step_inputs(B, H, torch.float32, seed=821, step=t, device=DEV)
          for t in range(T)]
    douts = [torch.randn((B, H, 128), generator=gen, device=DEV) for _ in range(T)]
    dST = 0.1 * torch.randn((B, H, 128, 128), generator=gen, device=DEV)
    states = [S0.clone()]
    S = S0.clone()
    for x in xs:
        libkda.recurrent_step(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], S)
        states.append(S.clone())
    torch.cuda.synchronize()
    # oracle forward states (fp64) and reverse pass
    ostates = [host64(S0)]
    for x in xs:
        _, Sn = oracle.step(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(x["g"]),
                            host64(x["beta"]), x["scale"], ostates[-1])
        ostates.append(Sn)
    dS_gpu, dS_ref = dST.clone(), host64(dST)
    worst = 0.0
    for t in reversed(range(T)):
        x = xs[t]
        g_gpu = libkda.recurrent_step_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"],
                                          states[t], douts[t], dS_gpu)
        torch.cuda.synchronize()
        g_ref = oracle.step_backward(host64(x["q"]), host64(x["k"]), host64(x["v"]),
                                     host64(x["g"]), host64(x["beta"]), x["scale"], ostates[t],
                                     host64(douts[t]), dS_ref)
        dS_ref = g_ref[5]
        for a, b in zip(g_gpu, g_ref[:5]):
            worst = max(worst, rel(host64(a), b))
    worst = max(worst, rel(host64(dS_gpu), dS_ref))
    say(f"BPTT over {T} tokens: worst gradient error {worst:.1e} (dh0 {rel(host64(dS_gpu), dS_ref):.1e})")
    assert worst <= TOL


def test_step_bwd_in_place_and_deterministic():
    x = inputs(2, 4, seed=830)
    a = gpu_bwd(x)
    b = gpu_bwd(x)
    for u, w in zip(a, b):
        assert torch.equal(u, w)
    # dS_prev equals exp(g) times the gradient of the decayed state: with
    # dout = 0 and beta = 0 it is exactly exp(g) * dS_next, row by row
    x["dout"].zero_()
    x["beta"].zero_()
    got = gpu_bwd(x)
    want = torch.exp(x["g"])[..., None] * x["dS"]
    assert torch.allclose(got[5], want, rtol=1e-6, atol=0)
    assert not got[2].any().item() and not got[0].any().item()   # dv = dq = 0
