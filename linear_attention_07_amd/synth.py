"""Seeded synthetic inputs for the KDA workloads.

This module holds the input recipes only (distributions, shapes, seeds) and
none of the KDA arithmetic; both the GPU path's tests/benchmark and the fp64
oracle consume what it produces (the oracle reads back the exact stored
bytes).  The recipes:

  q, k ~ N(0, 1), then scaled to unit length per token and head (in fp32,
        before the cast to the storage type);
  v ~ N(0, 1);
  g = -5 * sigmoid(x - shift), x ~ N(0, 1), per channel (shift 4, or 6 for
        the million-token case's slower decay);
  beta = sigmoid(N(0, 1)), one scalar per token and head;
  initial state ~ N(0, sigma^2) per entry, sigma = 0.1 ("N(0, 0.01)" read as
        mean and variance), or zero.

For the short convolution in front of the attention (kda_chunk_fwd_conv):

  raw q, k, v ~ N(0, 1) per entry (the projections' outputs, not normalised:
        the convolution comes first);
  taps ~ U(-0.5, 0.5), i.e. +-1/sqrt(4) for 4 taps (a conv layer's usual
        initial range), [H, 128, 4] fp32 per tensor;
  conv state ~ N(0, 1) raw tokens [3, B, 3, H, 128], or none (zeros).

Random numbers come from torch's seeded generator on the target device and
are drawn block by block over tokens so that million-token inputs never need
an fp32 temporary of the whole tensor.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

HEAD_DIM = 128


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill", "decode" or "prefill_bwd"
    B: int
    H: int
    T: int               # tokens (prefill) or decode steps
    io: torch.dtype      # q, k, v, o storage type
    seed: int
    g_shift: float = 4.0
    h0_std: float = 0.0

    @property
    def scale(self) -> float:
        return HEAD_DIM ** -0.5


WORKLOADS = {
    # B=1, H=2, T=256, fp32 in and out, zero initial state, both paths
    "small_f32": Workload("small_f32", "prefill", 1, 2, 256, torch.float32, 0),
    # one K3-shaped layer: 96 heads, 4K tokens, bf16 q/k/v, zero state
    "layer_4k": Workload("layer_4k", "prefill", 1, 96, 4096, torch.bfloat16, 1),
    # 64K-token prefill with a random initial state
    "prefill_64k": Workload("prefill_64k", "prefill", 1, 96, 65536, torch.bfloat16, 2,
                            h0_std=0.1),
    # 256 sequences x 96 heads, 64 decode steps, random initial state
    "decode_b256": Workload("decode_b256", "decode", 256, 96, 64, torch.bfloat16, 3,
                            h0_std=0.1),
    # backward of one fp32 layer prefill at a training length: 8K tokens, 96
    # heads, random initial state (dout and dhT drawn beside it)
    "prefill_bwd_8k": Workload("prefill_bwd_8k", "prefill_bwd", 1, 96, 8192, torch.float32, 5,
                               h0_std=0.1),
    # million-token prefill with slow decay, zero state
    "prefill_1m": Workload("prefill_1m", "prefill", 1, 96, 1 << 20, torch.bfloat16, 4,
                           g_shift=6.0),
}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _unit(x):
    return x / x.norm(dim=-1, keepdim=True)


def prefill_inputs(B, T, H, io=torch.bfloat16, seed=0, g_shift=4.0, h0_std=0.0,
                   device="cuda", block=16384):
    """q, k, v, g: [B, T, H, 128]; beta: [B, T, H]; h0: [B, H, 128, 128] or None."""
    dev = torch.device(device)
    gen = _gen(dev, seed)
    shp = (B, T, H, HEAD_DIM)
    q = torch.empty(shp, dtype=io, device=dev)
    k = torch.empty(shp, dtype=io, device=dev)
    v = torch.empty(shp, dtype=io, device=dev)
    g = torch.empty(shp, dtype=torch.float32, device=dev)
    beta = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    for t0 in range(0, T, block):
        tb = min(block, T - t0)
        bs = (B, tb, H, HEAD_DIM)
        q[:, t0:t0 + tb] = _unit(torch.randn(bs, generator=gen, device=dev)).to(io)
        k[:, t0:t0 + tb] = _unit(torch.randn(bs, generator=gen, device=dev)).to(io)
        v[:, t0:t0 + tb] = torch.randn(bs, generator=gen, device=dev).to(io)
        g[:, t0:t0 + tb] = -5.0 * torch.sigmoid(torch.randn(bs, generator=gen, device=dev) - g_shift)
        beta[:, t0:t0 + tb] = torch.sigmoid(torch.randn((B, tb, H), generator=gen, device=dev))
    h0 = None
    if h0_std > 0:
        h0 = torch.randn((B, H, HEAD_DIM, HEAD_DIM), generator=gen, device=dev) * h0_std
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, scale=HEAD_DIM ** -0.5)


def decode_state(B, H, seed, h0_std=0.1, device="cuda"):
    dev = torch.device(device)
    gen = _gen(dev, seed)
    return torch.randn((B, H, HEAD_DIM, HEAD_DIM), generator=gen, device=dev) * h0_std


def decode_step_inputs(B, H, io=torch.bfloat16, seed=0, step=0, g_shift=4.0, device="cuda"):
    """Fresh q, k, v [B, H, 128], g [B, H, 128], beta [B, H] for one step."""
    dev = torch.device(device)
    gen = _gen(dev, 1_000_003 * (int(seed) + 1) + int(step))
    shp = (B, H, HEAD_DIM)
    q = _unit(torch.randn(shp, generator=gen, device=dev)).to(io)
    k = _unit(torch.randn(shp, generator=gen, device=dev)).to(io)
    v = torch.randn(shp, generator=gen, device=dev).to(io)
    g = -5.0 * torch.sigmoid(torch.randn(shp, generator=gen, device=dev) - g_shift)
    beta = torch.sigmoid(torch.randn((B, H), generator=gen, device=dev))
    return dict(q=q, k=k, v=v, g=g, beta=beta, scale=HEAD_DIM ** -0.5)


def workload_inputs(w: Workload, device="cuda"):
    if w.kind != "prefill":
        raise ValueError("decode workloads are drawn per step with decode_step_inputs")
    return prefill_inputs(w.B, w.T, w.H, w.io, w.seed, w.g_shift, w.h0_std, device)


def conv_inputs(B, T, H, seed=0, with_state=True, h0_std=0.1, device="cuda", g_shift=4.0):
    """Inputs of the attention with its short convolution: raw q, k, v
    [B, T, H, 128] bf16; wq, wk, wv [H, 128, 4] fp32; conv_in
    [3, B, 3, H, 128] bf16 or None; g, beta, h0, scale as prefill_inputs."""
    inp = prefill_inputs(B, T, H, torch.bfloat16, seed, g_shift=g_shift, h0_std=h0_std,
                         device=device)
    dev = torch.device(device)
    gen = _gen(dev, 7_919 * (int(seed) + 1) + 17)
    shp = (B, T, H, HEAD_DIM)
    for name in ("q", "k", "v"):
        inp[name] = torch.randn(shp, generator=gen, device=dev).to(torch.bfloat16)
    for name in ("wq", "wk", "wv"):
        inp[name] = torch.rand((H, HEAD_DIM, 4), generator=gen, device=dev) - 0.5
    inp["conv_in"] = None
    if with_state:
        inp["conv_in"] = torch.randn((3, B, 3, H, HEAD_DIM), generator=gen,
                                     device=dev).to(torch.bfloat16)
    return inp


def decode_conv_inputs(B, H, seed=0, step=0, device="cuda"):
    """One decode token before its short convolution: raw q, k, v [B, H, 128]
    bf16 ~ N(0, 1); g, beta, scale as decode_step_inputs."""
    inp = decode_step_inputs(B, H, torch.bfloat16, seed, step, device=device)
    dev = torch.device(device)
    gen = _gen(dev, 7_919 * (int(seed) + 1) + 104_729 * (int(step) + 1) + 29)
    for name in ("q", "k", "v"):
        inp[name] = torch.randn((B, H, HEAD_DIM), generator=gen, device=dev).to(torch.bfloat16)
    return inp


def conv_params(B, H, seed=0, device="cuda"):
    """Taps wq, wk, wv [H, 128, 4] fp32 ~ U(-0.5, 0.5) and a conv state
    [3, B, 3, H, 128] bf16 ~ N(0, 1)."""
    dev = torch.device(device)
    gen = _gen(dev, 7_919 * (int(seed) + 1) + 31)
    out = {name: torch.rand((H, HEAD_DIM, 4), generator=gen, device=dev) - 0.5
           for name in ("wq", "wk", "wv")}
    out["conv_state"] = torch.randn((3, B, 3, H, HEAD_DIM), generator=gen,
                                    device=dev).to(torch.bfloat16)
    return out


def gate_logits(shape, seed=0, device="cuda"):
    """Logits of the output gate ~ N(0, 1), bf16, of the given shape
    ([B, T, H, 128] for a prefill, [B, H, 128] for a decode step)."""
    dev = torch.device(device)
    gen = _gen(dev, 7_919 * (int(seed) + 1) + 43)
    return torch.randn(tuple(shape), generator=gen, device=dev).to(torch.bfloat16)
