"""Million-token prefill (B=1, H=96, T=1,048,576, bf16 q/k/v, slow decay
g = -5 sigmoid(x - 6)) with all inputs resident on the device (about 155 GB).

The fp64 oracle follows all 96 heads over the whole length, streamed in
segments of 32,768 tokens with the state carried between them: the outputs of
heads 0 and 47 are compared at every token and the final state of every head
is compared.  The outputs of the other heads are covered by a property that
holds at any size: with beta = 1 and q = k every output equals scale * v.
"""
import numpy as np
import pytest
import torch

from kda_check import TOL_BF16, host64, oracle_threads, rel_state, say
from linear_attention_07_amd import libkda, synth
from oracle import oracle

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda"
OUT_HEADS = (0, 47)


@pytest.fixture(scope="module")
def million():
    w = synth.WORKLOADS["prefill_1m"]
    torch.cuda.empty_cache()   # blocks cached by earlier tests in this process
    free, total = torch.cuda.mem_get_info()
    if free < 170e9:
        pytest.skip(f"needs ~170 GB of device memory, {free / 1e9:.0f} GB free")
    say(f"generating {w}")
    inp = synth.workload_inputs(w, DEV)
    yield w, inp
    del inp
    torch.cuda.empty_cache()


@pytest.mark.timeout(1200)
def test_prefill_1m_against_oracle(million):
    w, inp = million
    out, hT = libkda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"])
    torch.cuda.synchronize()
    say("GPU done; streaming the oracle over all 96 heads")
    seg = 1 << 15
    S = None
    err = {h: 0.0 for h in OUT_HEADS}
    ref = {h: 0.0 for h in OUT_HEADS}
    for t0 in range(0, w.T, seg):
        t1 = min(w.T, t0 + seg)

        def seqs(x):  # [1, t, H, D] on the device -> [H, t, D] on the host
            return x[0, t0:t1].transpose(0, 1).contiguous().cpu()

        o_ref, S = oracle.run_sequences(seqs(inp["q"]), seqs(inp["k"]), seqs(inp["v"]),
                                        seqs(inp["g"]), inp["beta"][0, t0:t1].t().contiguous().cpu(),
                                        inp["scale"], S, threads=oracle_threads())
        for h in OUT_HEADS:
            got = out[0, t0:t1, h].to(torch.float64).cpu().numpy()
            err[h] = max(err[h], float(np.abs(got - o_ref[h]).max()))
            ref[h] = max(ref[h], float(np.abs(o_ref[h]).max()))
        if (t1 // seg) % 4 == 0 or t1 == w.T:
            say(f"  tokens {t1}: head0 {err[0] / ref[0]:.2e} head47 {err[47] / ref[47]:.2e}")
    eo = max(err[h] / ref[h] for h in err)
    es = rel_state(host64(hT), S.reshape(1, w.H, 128, 128))
    say(f"1M: out err (heads 0, 47) {eo:.2e}; final-state err (all 96 heads) {es:.2e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_prefill_1m_exact_recall_all_heads(million):
    w, inp = million
    ones = torch.ones_like(inp["beta"])
    out, _ = libkda.chunk_fwd(inp["k"], inp["k"], inp["v"], inp["g"], ones, inp["scale"],
                              final_state=False)
    torch.cuda.synchronize()
    worst = 0.0
    for t0 in range(0, w.T, 1 << 16):
        sl = slice(t0, t0 + (1 << 16))
        want = inp["scale"] * inp["v"][:, sl].float()
        d = (out[:, sl].float() - want).abs().amax(dim=(0, 1, 3))
        worst = max(worst, float((d / want.abs().amax(dim=(0, 1, 3))).max()))
    say(f"1M beta=1 recall, all 96 heads: {worst:.2e}")
    assert worst <= TOL_BF16
