"""kda_chunk_fwd_noalloc (the prefill for callers that cannot allocate: its
records and carried state live in the library's fixed per-GPU scratch) against
kda_chunk_fwd through the C-ABI: two calls in a row, the second smaller, each
bitwise equal to the allocating entry point (the same kernels; segmentation is
exact), plus an oracle check of the first."""
import pytest
import torch

from kda_check import TOL_BF16, host64, oracle_prefill, rel_out, rel_state, say
from linear_attention_07_amd import libkda, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def both(inp, h0, with_hT=True):
    B, T, H, _ = inp["q"].shape
    o1, h1 = libkda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"],
                              h0, final_state=with_hT)
    out = torch.empty_like(inp["v"])
    hT = torch.empty((B, H, 128, 128), device=DEV) if with_hT else None
    o2, h2 = libkda.chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                      inp["scale"], h0, out, hT)
    torch.cuda.synchronize()
    return o1, h1, o2, h2


def test_noalloc_two_calls_match_the_allocating_entry_point():
    # 1000 tokens x 96 heads: 16 chunk records of 96 heads exceed the scratch,
    # so this call runs in segments with the state carried in the scratch
    inp = synth.prefill_inputs(1, 1000, 96, torch.bfloat16, seed=81, h0_std=0.1, device=DEV)
    say("noalloc call 1: B=1 T=1000 H=96")
    o1, h1, o2, h2 = both(inp, inp["h0"])
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    o_ref, h_ref = oracle_prefill(inp, heads=[0, 95])
    eo = rel_out(host64(o2[:, :, [0, 95]]), o_ref)
    es = rel_state(host64(h2[:, [0, 95]]), h_ref)
    say(f"  vs oracle heads 0, 95: out {eo:.2e} state {es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    # a smaller second call: one segment, no initial state, no final state
    inp2 = synth.prefill_inputs(2, 130, 3, torch.bfloat16, seed=82, device=DEV)
    say("noalloc call 2: B=2 T=130 H=3")
    o1, _, o2, _ = both(inp2, None, with_hT=False)
    assert torch.equal(o1, o2)
    # and once more with the state carried in place (hT = h0)
    inp3 = synth.prefill_inputs(2, 200, 3, torch.bfloat16, seed=83, h0_std=0.1, device=DEV)
    o1, h1 = libkda.chunk_fwd(inp3["q"], inp3["k"], inp3["v"], inp3["g"], inp3["beta"],
                              inp3["scale"], inp3["h0"])
    S = inp3["h0"].clone()
    out = torch.empty_like(inp3["v"])
    libkda.chunk_fwd_noalloc(inp3["q"], inp3["k"], inp3["v"], inp3["g"], inp3["beta"],
                             inp3["scale"], S, out, S)
    torch.cuda.synchronize()
    assert torch.equal(o1, out) and torch.equal(h1, S)


def test_noalloc_rejects_what_does_not_fit():
    # 4200 heads: one chunk's records (16 KB per head) exceed the 64 MiB scratch
    inp = synth.prefill_inputs(1, 64, 4200, torch.bfloat16, seed=84, device=DEV)
    out = torch.empty_like(inp["v"])
    with pytest.raises(libkda.KDAError) as e:
        libkda.chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                 inp["scale"], None, out, None)
    assert e.value.status == libkda.KDA_ERR_UNSUPPORTED
