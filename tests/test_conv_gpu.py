"""GPU parity of kda_chunk_fwd_conv and kda_recurrent_step_conv (the 4-tap
short convolution + SiLU in front of the attention, fused into the prefill's
and the decode step's loads) against the fp64 oracle, through the C-ABI; plus
the conv state hand-over from prefill to decode, and edge cases.

The library rounds the filtered q, k, v to bf16 before the attention (its
documented input type).  Most comparisons give the oracle the same rounding
(round_bf16_inputs), so that they measure the kernels, as with plain bf16
inputs; where the fp32 filter of the library and the fp64 filter of the
oracle fall on either side of a bf16 rounding boundary the two inputs differ
by one bf16 ulp, on a few entries in 10^4.  The *_unrounded tests compare the
whole layer with the oracle's plain fp64 filter, no rounding anywhere, at the
same 1e-2 bar: the bf16 rounding of the filtered values is then counted as
error too.
"""
import os

import numpy as np
import pytest
import torch

from kda_check import TOL_BF16, host64, oracle_threads, rel_out, rel_state, say
from linear_attention_07_amd import libkda, synth
from oracle import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run(inp, conv_in="inp", h0="inp", **kw):
    ci = inp["conv_in"] if conv_in == "inp" else conv_in
    h = inp["h0"] if h0 == "inp" else h0
    out, hT, cout = libkda.chunk_fwd_conv(inp["q"], inp["k"], inp["v"], inp["wq"], inp["wk"],
                                          inp["wv"], inp["g"], inp["beta"], inp["scale"], h0=h,
                                          conv_in=ci, **kw)
    torch.cuda.synchronize()
    return out, hT, cout


def oracle_conv(inp, gate=None, rounded=True):
    ci = inp["conv_in"]
    cs = None if ci is None else tuple(host64(ci[i]) for i in range(3))
    h0 = inp["h0"]
    return oracle.forward_conv(host64(inp["q"]), host64(inp["k"]), host64(inp["v"]),
                               host64(inp["wq"]), host64(inp["wk"]), host64(inp["wv"]),
                               host64(inp["g"]), host64(inp["beta"]), inp["scale"],
                               None if h0 is None else host64(h0), cs, threads=oracle_threads(),
                               round_bf16_inputs=rounded,
                               gate=None if gate is None else host64(gate))


def sub(inp, t0, t1):
    return {k_: (v_[:, t0:t1].contiguous() if k_ in ("q", "k", "v", "g", "beta") else v_)
            for k_, v_ in inp.items()}


@pytest.mark.parametrize("B,T,H,state", [(2, 1, 3, True), (2, 3, 3, False), (2, 5, 3, True),
                                         (2, 65, 3, True), (2, 1000, 3, False),
                                         (1, 700, 8, True)])
def test_conv_against_oracle(B, T, H, state):
    inp = synth.conv_inputs(B, T, H, seed=500 + T + H, with_state=state, device=DEV)
    say(f"conv B={B} T={T} H={H} state={state}")
    out, hT, cout = run(inp)
    o_ref, h_ref, c_ref = oracle_conv(inp)
    eo, es = rel_out(host64(out), o_ref), rel_state(host64(hT), h_ref)
    say(f"  out err {eo:.2e} state err {es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    for i in range(3):   # raw tokens: exact
        assert np.array_equal(host64(cout[i]), c_ref[i]), i


def test_conv_layer_4k_all_heads():
    """One 96-head layer, T = 4096, with the convolution: every head checked."""
    B, T, H = 1, 4096, 96
    inp = synth.conv_inputs(B, T, H, seed=541, with_state=True, h0_std=0.0, device=DEV)
    out, hT, cout = run(inp)
    o_ref, h_ref, _ = oracle_conv(inp)
    eo, es = rel_out(host64(out), o_ref), rel_state(host64(hT), h_ref)
    say(f"conv layer_4k: out err {eo:.2e} state err {es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("B,T,H,state", [(2, 1, 3, True), (2, 65, 3, True), (2, 1000, 3, False),
                                         (1, 700, 8, True)])
def test_conv_against_unrounded_oracle(B, T, H, state):
    """The layer against the oracle's plain fp64 filter (no bf16 rounding of
    the filtered q, k, v on the oracle's side): ragged lengths, with and
    without a carried conv state."""
    inp = synth.conv_inputs(B, T, H, seed=560 + T + H, with_state=state, device=DEV)
    out, hT, cout = run(inp)
    o_ref, h_ref, c_ref = oracle_conv(inp, rounded=False)
    eo, es = rel_out(host64(out), o_ref), rel_state(host64(hT), h_ref)
    say(f"conv unrounded B={B} T={T} H={H} state={state}: out err {eo:.2e} state err {es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    for i in range(3):
        assert np.array_equal(host64(cout[i]), c_ref[i]), i


def test_gated_conv_layer_4k_all_heads_unrounded():
    """The whole layer (filter + attention + output gate), one 96-head layer
    at T = 4096 with a carried conv state, every head against the unrounded
    fp64 oracle."""
    B, T, H = 1, 4096, 96
    inp = synth.conv_inputs(B, T, H, seed=561, with_state=True, h0_std=0.1, device=DEV)
    z = synth.gate_logits((B, T, H, 128), seed=562, device=DEV)
    out, hT, _ = run(inp, gate=z)
    o_ref, h_ref, _ = oracle_conv(inp, gate=z, rounded=False)
    eo, es = rel_out(host64(out), o_ref), rel_state(host64(hT), h_ref)
    say(f"gated conv layer_4k unrounded: out err {eo:.2e} state err {es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_gated_decode_b256_unrounded():
    """The batched decode shape behind the filter and the gate, four steps,
    every output and state against the unrounded fp64 oracle."""
    B, H = 256, 96
    p = synth.conv_params(B, H, seed=630, device=DEV)
    S = synth.decode_state(B, H, seed=631, h0_std=0.1, device=DEV)
    S_ref = host64(S)
    for step in range(4):
        x = synth.decode_conv_inputs(B, H, seed=632, step=step, device=DEV)
        z = synth.gate_logits((B, H, 128), seed=633 + step, device=DEV)
        o_ref, S_ref, _ = decode_conv_oracle(x, p, S_ref, gate=z, rounded=False)
        out = libkda.recurrent_step_conv(x["q"], x["k"], x["v"], p["wq"], p["wk"], p["wv"],
                                         p["conv_state"], x["g"], x["beta"], x["scale"], S,
                                         gate=z)
        torch.cuda.synchronize()
        eo = rel_out(host64(out)[:, None], o_ref[:, None])
        say(f"gated decode b256 unrounded step {step}: out err {eo:.2e}")
        assert eo <= TOL_BF16
    es = rel_state(host64(S), S_ref)
    say(f"  state err {es:.2e}")
    assert es <= TOL_BF16


@pytest.mark.parametrize("split", [320, 100, 2])
def test_conv_chaining_matches_one_call(split):
    """T1 tokens, then T2 tokens from the returned attention state and conv
    state, equal one call over T1 + T2 tokens; bit for bit when the split is
    a chunk boundary."""
    B, T, H = 2, 640, 3
    inp = synth.conv_inputs(B, T, H, seed=543, with_state=True, device=DEV)
    out, hT, cout = run(inp)
    a, b = sub(inp, 0, split), sub(inp, split, T)
    oa, ha, ca = run(a)
    ob, hb, cb = run(b, conv_in=ca, h0=ha)
    o2 = torch.cat([oa, ob], dim=1)
    assert torch.equal(cb, cout)
    if split % 64 == 0:
        assert torch.equal(o2, out) and torch.equal(hb, hT)
    eo, es = rel_out(host64(o2), host64(out)), rel_state(host64(hb), host64(hT))
    say(f"conv chaining at {split}: out {eo:.2e} state {es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_conv_segmented_workspace_matches():
    """Workspace segments read the tokens before their first chunk from the
    raw inputs, and the gate by global token index: the split run equals the
    single-segment run exactly."""
    B, T, H = 1, 2000, 3
    inp = synth.conv_inputs(B, T, H, seed=544, with_state=True, device=DEV)
    z = synth.gate_logits((B, T, H, 128), seed=545, device=DEV)
    out1, h1, c1 = run(inp, gate=z)
    old = os.environ.get("KDA_WORKSPACE_MB")
    os.environ["KDA_WORKSPACE_MB"] = "1"
    try:
        out2, h2, c2 = run(inp, gate=z)
    finally:
        if old is None:
            del os.environ["KDA_WORKSPACE_MB"]
        else:
            os.environ["KDA_WORKSPACE_MB"] = old
    assert torch.equal(out1, out2) and torch.equal(h1, h2) and torch.equal(c1, c2)


def test_conv_state_in_place_and_optional():
    B, T, H = 2, 130, 3
    inp = synth.conv_inputs(B, T, H, seed=545, with_state=True, device=DEV)
    out, hT, cout = run(inp)
    st = inp["conv_in"].clone()
    out2, hT2, c2 = run(inp, conv_in=st, conv_out=st)          # updated in place
    assert c2 is st and torch.equal(st, cout)
    assert torch.equal(out2, out) and torch.equal(hT2, hT)
    out3, hT3, c3 = run(inp, final_state=False, final_conv=False)
    assert hT3 is None and c3 is None and torch.equal(out3, out)


def test_conv_short_and_empty():
    """T < 3 keeps part of the previous state; T = 0 passes it through (zeros
    for a fresh sequence)."""
    B, H = 2, 3
    inp = synth.conv_inputs(B, 2, H, seed=546, with_state=True, device=DEV)
    _, _, cout = run(inp)
    ci = inp["conv_in"]
    for i, name in enumerate(("q", "k", "v")):
        assert torch.equal(cout[i][:, 0], ci[i][:, 2])
        assert torch.equal(cout[i][:, 1:], inp[name][:, 0:2])
    e = synth.conv_inputs(B, 0, H, seed=547, with_state=True, device=DEV)
    out, hT, c0 = run(e)
    assert out.numel() == 0 and torch.equal(c0, e["conv_in"]) and torch.equal(hT, e["h0"])
    out, hT, c0 = run(e, conv_in=None, h0=None)
    assert not c0.any().item() and not hT.any().item()


def test_conv_filtered_values_match_oracle_closely():
    """With beta = 1 and the same taps for q and k, each read-out returns
    scale * v'_t, the filtered v (rounded to bf16): a direct check of the
    fused convolution + SiLU on v against the oracle's short convolution."""
    B, T, H = 1, 300, 4
    inp = synth.conv_inputs(B, T, H, seed=548, with_state=True, device=DEV)
    inp["k"] = inp["q"].clone()
    inp["wk"] = inp["wq"].clone()
    inp["conv_in"][1] = inp["conv_in"][0]
    inp["beta"] = torch.ones_like(inp["beta"])
    out, _, _ = run(inp)
    vf, _ = oracle.short_conv_silu(host64(inp["v"]), host64(inp["wv"]), host64(inp["conv_in"][2]),
                                   round_out=True)
    want = inp["scale"] * vf
    err = np.abs(host64(out) - want).max() / np.abs(want).max()
    say(f"conv recall: {err:.2e}")
    assert err <= TOL_BF16


def decode_conv_oracle(x, p, S, gate=None, rounded=True):
    cs = tuple(host64(p["conv_state"][i]) for i in range(3))
    return oracle.step_conv(host64(x["q"]), host64(x["k"]), host64(x["v"]), host64(p["wq"]),
                            host64(p["wk"]), host64(p["wv"]), cs, host64(x["g"]),
                            host64(x["beta"]), x["scale"], S, threads=oracle_threads(),
                            round_bf16_inputs=rounded,
                            gate=None if gate is None else host64(gate))


@pytest.mark.parametrize("B,H", [(3, 5), (2, 8)])
def test_decode_conv_against_oracle(B, H):
    """Four decode steps with fresh raw tokens, the conv state and the
    attention state carried on the device; B * H = 15 leaves the last
    workgroup half empty."""
    p = synth.conv_params(B, H, seed=600 + B, device=DEV)
    S = synth.decode_state(B, H, seed=601, h0_std=0.1, device=DEV)
    S_ref = host64(S)
    for step in range(4):
        x = synth.decode_conv_inputs(B, H, seed=602, step=step, device=DEV)
        o_ref, S_ref, cs_ref = decode_conv_oracle(x, p, S_ref)
        out = libkda.recurrent_step_conv(x["q"], x["k"], x["v"], p["wq"], p["wk"], p["wv"],
                                         p["conv_state"], x["g"], x["beta"], x["scale"], S)
        torch.cuda.synchronize()
        eo = rel_out(host64(out)[:, None], o_ref[:, None])
        say(f"decode conv B={B} H={H} step {step}: out err {eo:.2e}")
        assert eo <= TOL_BF16
        for i in range(3):   # raw tokens: exact
            assert np.array_equal(host64(p["conv_state"][i]), cs_ref[i]), (step, i)
    es = rel_state(host64(S), S_ref)
    say(f"  state err {es:.2e}")
    assert es <= TOL_BF16


def test_prefill_then_decode_conv():
    """A prefill over T tokens followed by decode steps from its attention
    and conv states equals one prefill over all the tokens."""
    B, T, H, n = 2, 130, 3, 5
    inp = synth.conv_inputs(B, T + n, H, seed=610, with_state=True, device=DEV)
    out_all, h_all, c_all = run(inp)
    out_a, S, cs = run(sub(inp, 0, T))
    outs = []
    for t in range(T, T + n):
        outs.append(libkda.recurrent_step_conv(
            inp["q"][:, t].contiguous(), inp["k"][:, t].contiguous(), inp["v"][:, t].contiguous(),
            inp["wq"], inp["wk"], inp["wv"], cs, inp["g"][:, t].contiguous(),
            inp["beta"][:, t].contiguous(), inp["scale"], S))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1)
    assert torch.equal(cs, c_all)
    eo = rel_out(host64(o_dec), host64(out_all[:, T:]))
    es = rel_state(host64(S), host64(h_all))
    say(f"prefill {T} + decode {n}: out {eo:.2e} state {es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_decode_conv_b256_all_heads():
    """The batched decode shape (B = 256, H = 96) with the convolution: two
    steps, every output and every state checked."""
    B, H = 256, 96
    p = synth.conv_params(B, H, seed=620, device=DEV)
    S = synth.decode_state(B, H, seed=621, h0_std=0.1, device=DEV)
    S_ref = host64(S)
    for step in range(2):
        x = synth.decode_conv_inputs(B, H, seed=622, step=step, device=DEV)
        o_ref, S_ref, cs_ref = decode_conv_oracle(x, p, S_ref)
        out = libkda.recurrent_step_conv(x["q"], x["k"], x["v"], p["wq"], p["wk"], p["wv"],
                                         p["conv_state"], x["g"], x["beta"], x["scale"], S)
        torch.cuda.synchronize()
        eo = rel_out(host64(out)[:, None], o_ref[:, None])
        say(f"decode conv b256 step {step}: out err {eo:.2e}")
        assert eo <= TOL_BF16
        for i in range(3):
            assert np.array_equal(host64(p["conv_state"][i]), cs_ref[i]), (step, i)
    es = rel_state(host64(S), S_ref)
    say(f"  state err {es:.2e}")
    assert es <= TOL_BF16



# ---------------------------------------------------------------------------
# the output gate behind the attention (out = o * sigmoid(z))
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,T,H", [(2, 1, 3), (2, 130, 3), (1, 1000, 8)])
def test_gated_conv_against_oracle(B, T, H):
    inp = synth.conv_inputs(B, T, H, seed=700 + T, with_state=True, device=DEV)
    z = synth.gate_logits((B, T, H, 128), seed=701 + T, device=DEV)
    out, hT, cout = run(inp, gate=z)
    out0, hT0, _ = run(inp)
    assert torch.equal(hT, hT0)           # the gate touches the output only
    o_ref, h_ref, _ = oracle_conv(inp, gate=z)
    eo, es = rel_out(host64(out), o_ref), rel_state(host64(hT), h_ref)
    say(f"gated conv B={B} T={T} H={H}: out err {eo:.2e} state err {es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    # logits of 0 halve the ungated output (up to the bf16 rounding of each)
    half, _, _ = run(inp, gate=torch.zeros_like(z))
    d = (host64(half) - 0.5 * host64(out0))
    assert np.abs(d).max() <= 2.0 ** -8 * np.abs(host64(out0)).max()


def test_gated_decode_and_prefill_chaining():
    """Prefill over T tokens and decode steps after it, all gated, against
    the oracle and against one gated prefill over every token."""
    B, T, H, n = 2, 130, 3, 4
    inp = synth.conv_inputs(B, T + n, H, seed=710, with_state=True, device=DEV)
    z = synth.gate_logits((B, T + n, H, 128), seed=711, device=DEV)
    out_all, h_all, c_all = run(inp, gate=z)
    o_ref, h_ref, _ = oracle_conv(inp, gate=z)
    assert rel_out(host64(out_all), o_ref) <= TOL_BF16
    _, S, cs = run(sub(inp, 0, T), gate=z[:, :T].contiguous())
    outs = []
    for t in range(T, T + n):
        outs.append(libkda.recurrent_step_conv(
            inp["q"][:, t].contiguous(), inp["k"][:, t].contiguous(), inp["v"][:, t].contiguous(),
            inp["wq"], inp["wk"], inp["wv"], cs, inp["g"][:, t].contiguous(),
            inp["beta"][:, t].contiguous(), inp["scale"], S, gate=z[:, t].contiguous()))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1)
    eo = rel_out(host64(o_dec), o_ref[:, T:])
    es = rel_state(host64(S), h_ref)
    say(f"gated prefill {T} + decode {n} vs oracle: out {eo:.2e} state {es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16 and torch.equal(cs, c_all)


def test_gated_decode_b256():
    B, H = 256, 96
    p = synth.conv_params(B, H, seed=720, device=DEV)
    S = synth.decode_state(B, H, seed=721, h0_std=0.1, device=DEV)
    S_ref = host64(S)
    x = synth.decode_conv_inputs(B, H, seed=722, step=0, device=DEV)
    z = synth.gate_logits((B, H, 128), seed=723, device=DEV)
    o_ref, S_ref, _ = decode_conv_oracle(x, p, S_ref, gate=z)
    out = libkda.recurrent_step_conv(x["q"], x["k"], x["v"], p["wq"], p["wk"], p["wv"],
                                     p["conv_state"], x["g"], x["beta"], x["scale"], S, gate=z)
    torch.cuda.synchronize()
    eo, es = rel_out(host64(out)[:, None], o_ref[:, None]), rel_state(host64(S), S_ref)
    say(f"gated decode b256: out err {eo:.2e} state err {es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_gated_conv_more_scan_workgroups_than_cus():
    """The whole layer (filter + attention + gate) at B=3, H=96: 576 scan
    workgroups, run in rounds; every head against the oracle."""
    B, T, H = 3, 200, 96
    inp = synth.conv_inputs(B, T, H, seed=730, with_state=True, device=DEV)
    z = synth.gate_logits((B, T, H, 128), seed=731, device=DEV)
    out, hT, cout = run(inp, gate=z)
    o_ref, h_ref, c_ref = oracle_conv(inp, gate=z)
    eo, es = rel_out(host64(out), o_ref), rel_state(host64(hT), h_ref)
    say(f"gated conv B={B} T={T} H={H}: out err {eo:.2e} state err {es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    for i in range(3):
        assert np.array_equal(host64(cout[i]), c_ref[i]), i
