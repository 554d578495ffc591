"""The KDA_DEBUG_CHECKS mode on the GPU, through the C-ABI: its precondition
scan rejects a log-decay below the -5 bound that the pages give for the decay
gate (深入 Kimi-K3 thread, KDA paragraph; Kimi K3 架构全景 page, section 02) and
values that are not finite, before anything is launched; valid inputs give the
same bits as without the mode; and a bounded device wait that gives up is
reported as KDA_ERR_DEVICE.  That last path is forced from the host with a
spin limit of one poll, so every kernel still ends normally (its waits return
at once after the first one gives up, every index stays in bounds)."""
import pytest
import torch

from kda_check import say
from linear_attention_07_amd import libkda, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture
def debug(monkeypatch):
    monkeypatch.setenv("KDA_DEBUG_CHECKS", "1")
    return monkeypatch


def status_of(fn):
    try:
        fn()
        torch.cuda.synchronize()
    except libkda.KDAError as e:
        return e.status
    return libkda.KDA_OK


def prefill(inp, **kw):
    return libkda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"],
                            inp["h0"], **kw)


@pytest.mark.parametrize("io", [torch.bfloat16, torch.float32])
def test_valid_inputs_pass_and_match(io, monkeypatch):
    inp = synth.prefill_inputs(1, 300, 4, io, seed=61, h0_std=0.1, device=DEV)
    inp["g"][0, 7, 2, 5] = -5.0                       # the bound itself is allowed
    o1, h1 = prefill(inp)
    torch.cuda.synchronize()
    monkeypatch.setenv("KDA_DEBUG_CHECKS", "1")
    o2, h2 = prefill(inp)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_decay_below_the_bound_is_rejected(debug):
    inp = synth.prefill_inputs(1, 130, 3, torch.bfloat16, seed=62, h0_std=0.1, device=DEV)
    inp["g"][0, 77, 1, 100] = -5.01
    assert status_of(lambda: prefill(inp)) == libkda.KDA_ERR_PRECONDITION
    inp["g"][0, 77, 1, 100] = 0.01                      # above 0 as well
    assert status_of(lambda: prefill(inp)) == libkda.KDA_ERR_PRECONDITION
    g16 = inp["g"].to(torch.bfloat16)
    g16[0, 77, 1, 100] = -5.0625                        # exact in bf16
    st = status_of(lambda: libkda.chunk_fwd(inp["q"], inp["k"], inp["v"], g16, inp["beta"],
                                            inp["scale"], inp["h0"]))
    assert st == libkda.KDA_ERR_PRECONDITION
    x = synth.decode_step_inputs(2, 3, torch.bfloat16, seed=63, device=DEV)
    x["g"][1, 2, 0] = -5.01
    S = synth.decode_state(2, 3, seed=64, device=DEV)
    S0 = S.clone()
    st = status_of(lambda: libkda.recurrent_step(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                                 x["scale"], S))
    assert st == libkda.KDA_ERR_PRECONDITION
    assert torch.equal(S, S0)                          # nothing was launched


def test_non_finite_values_are_rejected(debug):
    inp = synth.prefill_inputs(1, 100, 2, torch.bfloat16, seed=65, h0_std=0.1, device=DEV)
    v = inp["v"].clone()
    inp["v"][0, 50, 1, 3] = float("nan")
    assert status_of(lambda: prefill(inp)) == libkda.KDA_ERR_PRECONDITION
    inp["v"] = v
    inp["beta"][0, 3, 0] = float("inf")
    assert status_of(lambda: prefill(inp)) == libkda.KDA_ERR_PRECONDITION


def test_backward_checks(debug):
    B, T, H = 1, 100, 2
    x = synth.prefill_inputs(B, T, H, torch.float32, seed=66, h0_std=0.1, device=DEV)
    dout = torch.randn((B, T, H, 128), device=DEV)
    run = lambda: libkda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], dout,
                                   h0=x["h0"])
    assert status_of(run) == libkda.KDA_OK
    x["g"][0, 99, 1, 127] = -6.0
    assert status_of(run) == libkda.KDA_ERR_PRECONDITION
    x["g"][0, 99, 1, 127] = -1.0
    dout[0, 0, 0, 0] = float("nan")
    assert status_of(run) == libkda.KDA_ERR_PRECONDITION


def test_a_wait_that_gives_up_is_reported(debug):
    """One poll per wait: the scan's first wait for a record gives up, every
    later wait returns at once, the kernel ends, and the host hears of it."""
    debug.setenv("KDA_DEBUG_SPIN_LIMIT", "1")
    inp = synth.prefill_inputs(1, 4096, 4, torch.bfloat16, seed=67, h0_std=0.1, device=DEV)
    say("debug: spin limit 1, T=4096 H=4")
    assert status_of(lambda: prefill(inp)) == libkda.KDA_ERR_DEVICE
    # the status words are cleared at the next call: a normal limit passes
    debug.delenv("KDA_DEBUG_SPIN_LIMIT")
    assert status_of(lambda: prefill(inp)) == libkda.KDA_OK


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_a_backward_scan_wait_that_gives_up_is_reported(debug, io):
    """The backward's state and gradient scans hand each chunk from their loader
    waves to their scan waves through bounded LDS waits too: with one poll per
    wait the first unready one gives up, the kernels end, and the call reports
    KDA_ERR_DEVICE; the next call with the normal limit passes."""
    debug.setenv("KDA_DEBUG_SPIN_LIMIT", "1")
    x = synth.prefill_inputs(1, 4096, 4, io, seed=68, h0_std=0.1, device=DEV)
    dout = torch.randn((1, 4096, 4, 128), device=DEV).to(io)
    run = lambda: libkda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], dout,
                                   h0=x["h0"])
    say(f"debug: spin limit 1, backward T=4096 H=4 {io}")
    assert status_of(run) == libkda.KDA_ERR_DEVICE
    debug.delenv("KDA_DEBUG_SPIN_LIMIT")
    assert status_of(run) == libkda.KDA_OK


def test_an_fp32_scan_wait_that_gives_up_is_reported(debug):
    """The fp32 prefill's scan (loader and scan waves, bounded LDS waits) reports
    a wait that gives up the same way."""
    debug.setenv("KDA_DEBUG_SPIN_LIMIT", "1")
    inp = synth.prefill_inputs(1, 4096, 4, torch.float32, seed=69, h0_std=0.1, device=DEV)
    say("debug: spin limit 1, fp32 prefill T=4096 H=4")
    assert status_of(lambda: prefill(inp)) == libkda.KDA_ERR_DEVICE
    debug.delenv("KDA_DEBUG_SPIN_LIMIT")
    assert status_of(lambda: prefill(inp)) == libkda.KDA_OK
