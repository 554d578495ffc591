"""GPU parity of kda_chunk_bwd_f32 / kda_chunk_bwd (backward of the chunked
prefill) against the fp64 oracle's sequence_backward: the recurrence run
forward keeping every state, then differentiated token by token in reverse
(the plain definition of the gradient, pinned to central differences of the
oracle's forward).  Nothing chunk-shaped sits in the reference.

fp32 arithmetic throughout.  fp32 I/O: the bar is the fp32-mode one, 1e-3
normalised max error per gradient (max |gpu - oracle| / max |oracle|).  bf16
q / k / v / dout (kda_chunk_bwd): the oracle reads the same bf16 values and dq,
dk, dv are rounded to bf16, so their bar is the bf16 one, 1e-2; dg, dbeta and
dh0 stay fp32 and keep 1e-3.  Cases
span several chunks with a ragged last one, strong and mild decays, a nonzero
initial state and final-state gradient, one-token and empty sequences."""
import numpy as np
import pytest
import torch

from kda_check import host64, oracle_threads, say
from linear_attention_07_amd import libkda, synth
from oracle import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-3
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def rel(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(x - ref).max() / (den if den > 0 else 1.0))


def inputs(B, T, H, seed, g_shift=4.0, h0_std=0.1, dhT_std=0.1, io=torch.float32):
    x = synth.prefill_inputs(B, T, H, io, seed=seed, g_shift=g_shift, h0_std=h0_std,
                             device=DEV)
    gen = torch.Generator(device=DEV).manual_seed(seed + 7)
    x["dout"] = torch.randn((B, T, H, 128), generator=gen, device=DEV).to(io)
    x["dhT"] = (dhT_std * torch.randn((B, H, 128, 128), generator=gen, device=DEV)
                if dhT_std > 0 else None)
    return x


def gpu(x):
    r = libkda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], x["dout"],
                         h0=x["h0"], dhT=x["dhT"])
    torch.cuda.synchronize()
    return r


def ref(x):
    h = lambda t: None if t is None else host64(t)
    return oracle.sequence_backward(h(x["q"]), h(x["k"]), h(x["v"]), h(x["g"]), h(x["beta"]),
                                    x["scale"], h(x["h0"]), h(x["dout"]), h(x["dhT"]),
                                    threads=oracle_threads())


def tol(name, io):
    return 1e-2 if io == torch.bfloat16 and name in ("dq", "dk", "dv") else TOL


def check(x, label):
    got = gpu(x)
    want = ref(x)
    io = x["q"].dtype
    errs = {n: rel(host64(a), b) for n, a, b in zip(NAMES, got, want)}
    say(f"chunk bwd {label}: " + " ".join(f"{n} {e:.1e}" for n, e in errs.items()))
    for n, a in zip(NAMES, got):
        assert torch.isfinite(a).all(), n
    for n, e in errs.items():
        assert e <= tol(n, io), (n, e)


@pytest.mark.parametrize("B,T,H,g_shift", [(1, 64, 1, 4.0), (1, 100, 2, 4.0), (2, 200, 3, 0.0),
                                           (1, 1, 1, 4.0), (1, 65, 1, -2.0)])
def test_chunk_bwd_against_oracle(B, T, H, g_shift):
    say(f"chunk bwd case B={B} T={T} H={H} g_shift={g_shift}")
    check(inputs(B, T, H, seed=900 + T + H, g_shift=g_shift), f"B={B} T={T} H={H} "
          f"g_shift={g_shift}")


@pytest.mark.parametrize("B,T,H,g_shift", [(1, 64, 1, 4.0), (2, 200, 3, 0.0), (1, 1, 1, 4.0),
                                           (1, 130, 2, -2.0)])
def test_chunk_bwd_bf16_against_oracle(B, T, H, g_shift):
    say(f"chunk bwd bf16 case B={B} T={T} H={H} g_shift={g_shift}")
    check(inputs(B, T, H, seed=700 + T + H, g_shift=g_shift, io=torch.bfloat16),
          f"bf16 B={B} T={T} H={H} g_shift={g_shift}")


def test_chunk_bwd_bf16_matches_fp32_on_the_same_values():
    """bf16 inputs widened to fp32 give the same gradients through both entry
    points (the same fp32 arithmetic), up to the bf16 rounding of dq, dk, dv."""
    x16 = inputs(1, 150, 2, seed=733, io=torch.bfloat16)
    x32 = {kk: (vv.float() if torch.is_tensor(vv) and vv.dtype == torch.bfloat16 else vv)
           for kk, vv in x16.items()}
    a, b = gpu(x16), gpu(x32)
    for n, u, w in zip(NAMES, a, b):
        e = rel(host64(u), host64(w))
        say(f"chunk bwd bf16 vs fp32 entry {n}: {e:.1e}")
        assert e <= (4e-3 if n in ("dq", "dk", "dv") else 1e-6), (n, e)


def test_chunk_bwd_zero_state_and_no_final_gradient():
    x = inputs(1, 130, 2, seed=931, h0_std=0.0, dhT_std=0.0)
    assert x["h0"] is None and x["dhT"] is None
    check(x, "h0 = dhT = 0")


def test_chunk_bwd_long_sequence():
    """4096 tokens (64 chunks) over 4 heads: the two state scans carry the
    state and its gradient across every chunk boundary."""
    say("chunk bwd case B=1 T=4096 H=4")
    check(inputs(1, 4096, 4, seed=977, g_shift=2.0), "B=1 T=4096 H=4")


def test_chunk_bwd_empty_sequence_passes_the_state_gradient():
    x = inputs(2, 0, 3, seed=5)
    dq, dk, dv, dg, dbeta, dh0 = gpu(x)
    assert dq.numel() == 0 and dbeta.numel() == 0
    assert torch.equal(dh0, x["dhT"])


def test_chunk_bwd_matches_chained_step_backward_on_gpu():
    """The chunkwise backward equals the GPU's own step backward chained over
    the states of the GPU's recurrent steps (two independent kernels)."""
    B, T, H = 1, 80, 2
    x = inputs(B, T, H, seed=951)
    got = gpu(x)
    S = x["h0"].clone()
    states = []
    for t in range(T):
        states.append(S.clone())
        out = torch.empty((B, H, 128), device=DEV)
        libkda.recurrent_step(x["q"][:, t].contiguous(), x["k"][:, t].contiguous(),
                              x["v"][:, t].contiguous(), x["g"][:, t].contiguous(),
                              x["beta"][:, t].contiguous(), x["scale"], S, out=out)
    dS = x["dhT"].clone()
    want = [torch.empty_like(x[n]) for n in ("q", "k", "v", "g", "beta")]
    for t in reversed(range(T)):
        r = libkda.recurrent_step_bwd(x["q"][:, t].contiguous(), x["k"][:, t].contiguous(),
                                      x["v"][:, t].contiguous(), x["g"][:, t].contiguous(),
                                      x["beta"][:, t].contiguous(), x["scale"], states[t],
                                      x["dout"][:, t].contiguous(), dS)
        for j in range(5):
            want[j][:, t] = r[j]
    torch.cuda.synchronize()
    for n, a, b in zip(NAMES, got, (*want, dS)):
        e = rel(host64(a), host64(b))
        say(f"chunk bwd vs chained steps {n}: {e:.1e}")
        assert e <= TOL, (n, e)


def test_chunk_bwd_deterministic():
    x = inputs(1, 150, 2, seed=961)
    a = gpu(x)
    b = gpu(x)
    for n, u, w in zip(NAMES, a, b):
        assert torch.equal(u, w), n


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_chunk_bwd_bench_workload_sampled_heads(io):
    """The timed workload (B=1, H=96, T=8192, as launched by the benchmark, with
    fp32 and with bf16 I/O): heads are independent, so the oracle runs on three
    sampled heads."""
    w = synth.WORKLOADS["prefill_bwd_8k"]
    say(f"chunk bwd case {w.name} B={w.B} T={w.T} H={w.H} {io}")
    x = synth.prefill_inputs(w.B, w.T, w.H, torch.float32, seed=w.seed, g_shift=w.g_shift,
                             h0_std=w.h0_std, device=DEV)
    gb = torch.Generator(device=DEV).manual_seed(w.seed + 1)
    x["dout"] = torch.randn((w.B, w.T, w.H, 128), generator=gb, device=DEV)
    x["dhT"] = 0.1 * torch.randn((w.B, w.H, 128, 128), generator=gb, device=DEV)
    for key in ("q", "k", "v", "dout"):
        x[key] = x[key].to(io)
    got = gpu(x)
    heads = [0, 47, w.H - 1]
    h = lambda t, ax: host64(t.index_select(ax, torch.tensor(heads, device=DEV)))
    want = oracle.sequence_backward(h(x["q"], 2), h(x["k"], 2), h(x["v"], 2), h(x["g"], 2),
                                    h(x["beta"], 2), x["scale"], h(x["h0"], 1),
                                    h(x["dout"], 2), h(x["dhT"], 1), threads=len(heads))
    axes = (2, 2, 2, 2, 2, 1)
    for n, a, b, ax in zip(NAMES, got, want, axes):
        e = rel(h(a, ax), b)
        say(f"chunk bwd {w.name} {io} heads {heads} {n}: {e:.1e}")
        assert e <= tol(n, io), (n, e)


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_chunk_bwd_segmented_workspace(io, monkeypatch):
    """A 1 MB workspace budget splits the call into one segment per chunk (a
    forward pass keeping each segment's entering state, then the segments
    differentiated last to first from their checkpoints, the state gradient
    carried between them): bitwise the one-segment result, and the oracle's."""
    x = inputs(2, 300, 2, seed=991, io=io)
    one = gpu(x)
    monkeypatch.setenv("KDA_WORKSPACE_MB", "1")
    many = gpu(x)
    for n, u, w in zip(NAMES, one, many):
        assert torch.equal(u, w), n
    check(x, f"{io} B=2 T=300 H=2 in 5 segments")
    x["dhT"] = None            # no final gradient, no initial state wanted
    r = libkda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], x["dout"],
                         h0=x["h0"], dhT=None)
    torch.cuda.synchronize()
    assert torch.isfinite(r[5]).all()


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_chunk_bwd_batched_heads(io):
    """B=2, H=8: B*H a multiple of 8, so both state scans take their XCD-aware
    workgroup order across two batch entries; ragged T=150."""
    check(inputs(2, 150, 8, seed=993, io=io), f"{io} B=2 T=150 H=8")


def test_chunk_bwd_64k_in_a_fixed_budget():
    """64K tokens x 96 heads (1024 chunks; about 27 GB of workspace in one
    segment) inside the default 8 GB budget: four segments.  Two heads checked
    in full against the token-by-token oracle."""
    B, T, H = 1, 65536, 96
    say(f"chunk bwd case B={B} T={T} H={H} fp32, default budget")
    x = synth.prefill_inputs(B, T, H, torch.float32, seed=993, g_shift=4.0, h0_std=0.1,
                             device=DEV)
    gb = torch.Generator(device=DEV).manual_seed(994)
    x["dout"] = torch.randn((B, T, H, 128), generator=gb, device=DEV)
    x["dhT"] = 0.1 * torch.randn((B, H, 128, 128), generator=gb, device=DEV)
    got = gpu(x)
    for n, a in zip(NAMES, got):
        assert torch.isfinite(a).all(), n
    heads = [0, H - 1]
    h = lambda t, ax: host64(t.index_select(ax, torch.tensor(heads, device=DEV)))
    want = oracle.sequence_backward(h(x["q"], 2), h(x["k"], 2), h(x["v"], 2), h(x["g"], 2),
                                    h(x["beta"], 2), x["scale"], h(x["h0"], 1),
                                    h(x["dout"], 2), h(x["dhT"], 1), threads=len(heads))
    for n, a, b, ax in zip(NAMES, got, want, (2, 2, 2, 2, 2, 1)):
        e = rel(h(a, ax), b)
        say(f"chunk bwd 64K heads {heads} {n}: {e:.1e}")
        assert e <= TOL, (n, e)
    libkda.trim_workspace()
