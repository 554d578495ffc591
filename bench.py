#!/usr/bin/env python3
"""Benchmark of the KDA forward pass on one MI355X.

A step is one kda_chunk_fwd over the 64K-token, 96-head prefill batch
(B=1, H=96, T=65536, d=128; bf16 q/k/v, fp32 g/beta, fp32 state with a
random initial state) with every input already resident in HBM.  The value is
prefill Mtok/s (B*T tokens per step, all 96 heads).  The same run also times
the same prefill with g in bf16 (kda_chunk_fwd_g16) and with the short
convolution in front and the output gate behind (kda_chunk_fwd_conv), the
batched decode step (B=256, H=96, fp32 state streamed in place; also with the
short convolution and the gate, kda_recurrent_step_conv) and reports its state bandwidth, and times the fp64
CPU oracle on a bounded sample of the prefill workload as a baseline.  It also
reports the other prefill workloads of the path: the latency in microseconds of
the small fp32 case (B=1, H=2, T=256) through both paths (one chunked call, and
256 decode steps), one 96-head layer at T=4096, and the million-token prefill
(B=1, H=96, T=1,048,576, about 155 GB resident), each with its HBM fraction
and the oracle timed on a labelled sample of it.

Roofline (per call of the timed op, algorithmic bytes only):
  prefill: 1540 B per token-head (q, k, v, o in bf16 = 4 x 256 B; g 512 B;
           beta 4 B) plus 64 KB of initial and 64 KB of final state per head;
  decode:  132,612 B per (sequence, head): the 64 KB state read and written,
           q, k, v (768 B), g (512 B), beta (4 B), o (256 B).
Both are HBM-bound (about 117 and 0.86 flop/B, under the 312 flop/B ridge
of 2.5 PFLOP/s bf16 over 8 TB/s), so the peak is 8 TB/s.  The prefill's
algorithmic matrix work, 180,224 flop per token-head at a fixed 64-token chunk
(five 64x64x128 products and three 128x128x64 state products), is reported
beside it as a fraction of the 2.5 PFLOP/s dense bf16 peak.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PREFILL_FLOP_PER_TOKEN_HEAD = 10 * 64 * 128 + 6 * 128 * 128
PREFILL_BYTES_PER_TOKEN_HEAD = 3 * 256 + 512 + 4 + 256
PREFILL_G16_BYTES_PER_TOKEN_HEAD = 3 * 256 + 256 + 4 + 256
STATE_BYTES = 128 * 128 * 4
DECODE_BYTES_PER_SEQ_HEAD = 2 * STATE_BYTES + 3 * 256 + 512 + 4 + 256
# the short convolution's state: 3 raw bf16 tokens of q, k and v per
# (sequence, head), read and written once per decode step; its taps
# (3 x [H, 128, 4] fp32) are read once per call
CONV_STATE_BYTES = 3 * 3 * 128 * 2
CONV_TAP_BYTES_PER_HEAD = 3 * 128 * 4 * 4
# the output gate's bf16 logits, one per output value
GATE_BYTES_PER_TOKEN_HEAD = 128 * 2
# backward of one fp32 decode step per (sequence, head): the state before the
# step and the state gradient read, the state gradient written; q, k, v, g,
# dout read and dq, dk, dv, dg written (fp32); beta read, dbeta written
BWD_STEP_BYTES_PER_SEQ_HEAD = 3 * STATE_BYTES + 9 * 128 * 4 + 2 * 4
# backward of the fp32 chunked prefill (kda_chunk_bwd_f32), algorithmic work
# per 64-token chunk and head, in units of one 64x64x128 product (MACs):
# record prep 4 (W, the two decayed key products P and N, M W); state scan 5
# (T V - W S, Kb^T Z); gradient scan 6 (Kb dS', W^T Y + Q'^T dO); chunk
# gradients 20 (R 2, U 1, dU 3, dR 1, dT 1, dM 1, X^T dX and its product
# with X^T 1, dQt dKt dKb 6, the pairwise-decay terms 4).  P and N count
# once: the chunk gradients read them from prep.
BWD_CHUNK_FLOP_PER_CHUNK_HEAD = int(2 * 35 * 64 * 64 * 128)
# its algorithmic HBM bytes per token-head: q, k, v, g, dout read and dq, dk,
# dv, dg written (fp32), beta read and dbeta written; per head h0 and dhT
# read, dh0 written
BWD_CHUNK_BYTES_PER_TOKEN_HEAD = 9 * 128 * 4 + 2 * 4
FP32_VALU_PEAK_TFLOPS = 157.3
# the same with bf16 q, k, v, dout in and dq, dk, dv out (g, dg fp32)
BWD_CHUNK_BF16_BYTES_PER_TOKEN_HEAD = 7 * 128 * 2 + 2 * 128 * 4 + 2 * 4


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="timed decode steps (default: the workload's 64 consecutive "
                         "steps, each with its own inputs)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (for profiler runs)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=65536)
    ap.add_argument("--only", default="all",
                    help="comma-separated workloads to run (prefill, prefill_g16, prefill_conv, "
                         "decode, decode_conv, decode_bwd, prefill_bwd, small_f32, layer_4k, "
                         "prefill_1m), for profiler passes; the default runs all; the headline "
                         "prefill always runs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed region, copy 1 GiB once (reference kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


# the sources the measured kernels and their launches are built from
MEASURED_SOURCES = ("kda_api.hip", "kda_bf16.hpp", "kda_chunk.hip", "kda_chunk16.hip",
                    "kda_chunk_bwd.hip", "kda_common.hpp", "kda_decode.hip", "kda_launch.hpp")


def kernel_sources_digest():
    """sha256 over the sources of the measured kernels: a traffic figure
    measured on other sources is not reported."""
    import hashlib
    d = hashlib.sha256()
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "linear_attention_07_amd", "csrc")
    for name in MEASURED_SOURCES:
        with open(os.path.join(src, name), "rb") as f:
            d.update(name.encode() + b"\0" + f.read())
    return d.hexdigest()


def measured_traffic(key):
    """HBM bytes per call from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != kernel_sources_digest():
        return None
    return rec.get(key, {}).get("bytes_per_call")


def time_op(torch, fn, steps, warmup):
    """Mean ms per call over `steps` calls bracketed by two events on the
    launch stream, and the median and minimum of the per-call event times."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return ev[0].elapsed_time(ev[steps]) / steps, per[len(per) // 2], per[0]


def oracle_sample(inp, heads, n_tokens):
    """Seconds of fp64 oracle time on the first n_tokens tokens of the given
    heads (all host threads)."""
    from oracle import oracle
    sel = torch_index(heads)

    def host(x):
        return x[:, :n_tokens][:, :, sel].detach().to("cpu").double().numpy()

    args = [host(inp[k]) for k in ("q", "k", "v", "g", "beta")]
    s0 = inp.get("h0")
    s0 = None if s0 is None else s0[:, sel].detach().to("cpu").double().numpy()
    t0 = time.perf_counter()
    oracle.forward(*args, inp["scale"], s0, threads=oracle.default_threads())
    return time.perf_counter() - t0


def torch_index(heads):
    import torch
    return torch.tensor(list(heads), dtype=torch.long)


def cpu_baseline(inp, n_tokens):
    """fp64 oracle on the same prefill input (first n_tokens tokens, every
    head), in groups of heads so that host memory stays bounded; all host
    threads, one head per thread at a time."""
    from oracle import oracle
    threads = oracle.default_threads()
    H = inp["q"].shape[2]
    t_sl = slice(0, n_tokens)
    group = max(1, 3 * threads)
    dt = 0.0
    for h0 in range(0, H, group):
        heads = slice(h0, min(H, h0 + group))

        def host(x):
            return x[:, t_sl, heads].detach().to("cpu").double().numpy()

        args = [host(inp[k]) for k in ("q", "k", "v", "g", "beta")]
        s0 = inp.get("h0")
        s0 = None if s0 is None else s0[:, heads].detach().to("cpu").double().numpy()
        t0 = time.perf_counter()
        oracle.forward(*args, inp["scale"], s0, threads=threads)
        dt += time.perf_counter() - t0
        del args, s0
    mtok = n_tokens / dt / 1e6
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": mtok, "unit": "Mtok/s", "cores": threads, "kind": "oracle", "cpu_model": model,
            "sample": f"all {H} heads x first {n_tokens} tokens of the 64K prefill input "
                      f"(the whole workload at the default), fp64 token-by-token recurrence, "
                      f"{dt:.2f} s of oracle time"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding of the path is a design note, not a run.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from linear_attention_07_amd import libkda, synth

    only = set(args.only.split(","))

    def want(name):
        return "all" in only or name in only

    libkda.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    res = {}

    def hbm(gbps, nbytes, **extra):
        r = {"bound": "hbm"}
        r.update(extra)
        r.update({"achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                  "frac": round(gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes_per_call": nbytes})
        return r

    def times(ms, ms_med, ms_min, nd=4):
        return {"ms_per_step": round(ms, nd), "ms_per_step_median": round(ms_med, nd),
                "ms_per_step_min": round(ms_min, nd)}

    # ---- prefill (the headline) -----------------------------------------------
    w = synth.WORKLOADS["prefill_64k"]
    inp = synth.workload_inputs(w, dev)
    out = torch.empty_like(inp["v"])
    hT = torch.empty((w.B, w.H, 128, 128), dtype=torch.float32, device=dev)

    def prefill():
        libkda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"],
                         inp["h0"], out=out, hT=hT)

    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    ms, ms_med, ms_min = time_op(torch, prefill, args.steps, args.warmup)
    t_wall = time.perf_counter() - t_wall0
    tokens = w.B * w.T
    mtok = tokens / (ms / 1e3) / 1e6
    token_heads = w.B * w.T * w.H
    pre_bytes = token_heads * PREFILL_BYTES_PER_TOKEN_HEAD + 2 * w.B * w.H * STATE_BYTES
    pre_gbps = pre_bytes / (ms / 1e3) / 1e9
    pre_tflops = token_heads * PREFILL_FLOP_PER_TOKEN_HEAD / (ms / 1e3) / 1e12
    print(f"# prefill: {ms:.3f} ms/step, {mtok:.2f} Mtok/s, {pre_gbps:.0f} GB/s algorithmic "
          f"(wall {t_wall:.2f} s)", file=sys.stderr, flush=True)

    # ---- prefill with g in bf16 ---------------------------------------------
    if want("prefill_g16"):
        g16 = inp["g"].to(torch.bfloat16)

        def prefill_g16():
            libkda.chunk_fwd(inp["q"], inp["k"], inp["v"], g16, inp["beta"], inp["scale"],
                             inp["h0"], out=out, hT=hT)

        t = time_op(torch, prefill_g16, args.steps, args.warmup)
        nb = token_heads * PREFILL_G16_BYTES_PER_TOKEN_HEAD + 2 * w.B * w.H * STATE_BYTES
        gb = nb / (t[0] / 1e3) / 1e9
        print(f"# prefill, bf16 g: {t[0]:.3f} ms/step, {tokens / (t[0] / 1e3) / 1e6:.2f} Mtok/s, "
              f"{gb:.0f} GB/s algorithmic", file=sys.stderr, flush=True)
        res["prefill_g16"] = {
            "workload": "prefill_64k with g in bf16 (kda_chunk_fwd_g16): 1,284 B per token-head",
            **times(*t), "Mtok_s": round(tokens / (t[0] / 1e3) / 1e6, 3), "roofline": hbm(gb, nb)}
        del g16

    # ---- prefill with the short convolution ---------------------------------
    if want("prefill_conv"):
        cp = synth.conv_params(w.B, w.H, seed=w.seed, device=dev)
        cout = torch.empty_like(cp["conv_state"])
        zg = synth.gate_logits(inp["v"].shape, seed=w.seed, device=dev)

        def prefill_conv():
            libkda.chunk_fwd_conv(inp["q"], inp["k"], inp["v"], cp["wq"], cp["wk"], cp["wv"],
                                  inp["g"], inp["beta"], inp["scale"], inp["h0"],
                                  conv_in=cp["conv_state"], conv_out=cout, out=out, hT=hT,
                                  gate=zg)

        t = time_op(torch, prefill_conv, args.steps, args.warmup)
        nb = pre_bytes + token_heads * GATE_BYTES_PER_TOKEN_HEAD + \
            w.B * w.H * 2 * CONV_STATE_BYTES + w.H * CONV_TAP_BYTES_PER_HEAD
        gb = nb / (t[0] / 1e3) / 1e9
        print(f"# prefill, short conv + gate: {t[0]:.3f} ms/step, "
              f"{tokens / (t[0] / 1e3) / 1e6:.2f} Mtok/s, {gb:.0f} GB/s algorithmic",
              file=sys.stderr, flush=True)
        res["prefill_conv"] = {
            "workload": "prefill_64k as one KDA layer: the 4-tap short convolution + SiLU on "
                        "q, k, v in front, the sigmoid output gate behind (kda_chunk_fwd_conv), "
                        "conv state in and out",
            **times(*t), "Mtok_s": round(tokens / (t[0] / 1e3) / 1e6, 3), "roofline": hbm(gb, nb)}
        del cp, cout, zg

    # ---- decode -------------------------------------------------------------
    wd = synth.WORKLOADS["decode_b256"]
    nbh = wd.B * wd.H
    dsteps = args.decode_steps or wd.T
    S = None
    if want("decode") or want("decode_conv"):
        S = synth.decode_state(wd.B, wd.H, seed=wd.seed, h0_std=wd.h0_std, device=dev)
    it = [0]
    if want("decode"):
        # the workload's 64 consecutive steps, each with its own inputs (drawn
        # beforehand); warm-up steps reuse the first ones
        xs = [synth.decode_step_inputs(wd.B, wd.H, wd.io, seed=wd.seed, step=t, device=dev)
              for t in range(dsteps)]
        dout = torch.empty_like(xs[0]["v"])

        def decode():
            x = xs[it[0] % dsteps]
            it[0] += 1
            libkda.recurrent_step(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"], S,
                                  out=dout)

        t = time_op(torch, decode, dsteps, args.warmup)
        del xs
        state_gbps = nbh * 2 * STATE_BYTES / (t[0] / 1e3) / 1e9
        dec_gbps = nbh * DECODE_BYTES_PER_SEQ_HEAD / (t[0] / 1e3) / 1e9
        print(f"# decode: {t[0]:.3f} ms/step, state {state_gbps:.0f} GB/s, "
              f"total {dec_gbps:.0f} GB/s", file=sys.stderr, flush=True)
        res["decode"] = {
            "workload": "decode_b256: B=256 H=96, fp32 state in place, bf16 q/k/v; 64 "
                        "consecutive steps timed, fresh inputs each step",
            **times(*t), "state_GBps": round(state_gbps, 1),
            "roofline": hbm(dec_gbps, nbh * DECODE_BYTES_PER_SEQ_HEAD, kernel="kda_decode_kernel",
                            traffic=measured_traffic("decode_b256"))}

    # ---- decode with the short convolution ----------------------------------
    if want("decode_conv"):
        dcp = synth.conv_params(wd.B, wd.H, seed=wd.seed, device=dev)
        xcs = [synth.decode_conv_inputs(wd.B, wd.H, seed=wd.seed, step=t, device=dev)
               for t in range(4)]
        zds = [synth.gate_logits((wd.B, wd.H, 128), seed=wd.seed + t, device=dev)
               for t in range(4)]
        dout = torch.empty((wd.B, wd.H, 128), dtype=torch.bfloat16, device=dev)

        def decode_conv():
            x, z = xcs[it[0] & 3], zds[it[0] & 3]
            it[0] += 1
            libkda.recurrent_step_conv(x["q"], x["k"], x["v"], dcp["wq"], dcp["wk"], dcp["wv"],
                                       dcp["conv_state"], x["g"], x["beta"], x["scale"], S,
                                       out=dout, gate=z)

        t = time_op(torch, decode_conv, dsteps, args.warmup)
        nb = nbh * (DECODE_BYTES_PER_SEQ_HEAD + 2 * CONV_STATE_BYTES +
                    GATE_BYTES_PER_TOKEN_HEAD) + wd.H * CONV_TAP_BYTES_PER_HEAD
        gb = nb / (t[0] / 1e3) / 1e9
        print(f"# decode, short conv + gate: {t[0]:.3f} ms/step, total {gb:.0f} GB/s",
              file=sys.stderr, flush=True)
        res["decode_conv"] = {
            "workload": "decode_b256 as one KDA layer: short convolution in front, output "
                        "gate behind (kda_recurrent_step_conv), conv state advanced in place",
            **times(*t), "roofline": hbm(gb, nb)}
        del dcp, xcs, zds
    del S

    # ---- backward of one decode step (fp32) ---------------------------------
    if want("decode_bwd"):
        xb = synth.decode_step_inputs(wd.B, wd.H, torch.float32, seed=wd.seed, step=0,
                                      device=dev)
        Sp = synth.decode_state(wd.B, wd.H, seed=wd.seed, h0_std=wd.h0_std, device=dev)
        dSb = synth.decode_state(wd.B, wd.H, seed=wd.seed + 1, h0_std=wd.h0_std, device=dev)
        dob = torch.randn((wd.B, wd.H, 128), device=dev)

        def decode_bwd():
            libkda.recurrent_step_bwd(xb["q"], xb["k"], xb["v"], xb["g"], xb["beta"],
                                      xb["scale"], Sp, dob, dSb)

        t = time_op(torch, decode_bwd, dsteps, args.warmup)
        nb = nbh * BWD_STEP_BYTES_PER_SEQ_HEAD
        gb = nb / (t[0] / 1e3) / 1e9
        print(f"# decode backward step: {t[0]:.3f} ms/step, total {gb:.0f} GB/s",
              file=sys.stderr, flush=True)
        res["decode_bwd"] = {
            "workload": "backward of one decode step at B=256 H=96, all fp32 "
                        "(kda_recurrent_step_bwd_f32): state and state gradient read, "
                        "state gradient written in place",
            **times(*t), "roofline": hbm(gb, nb)}
        del xb, Sp, dSb, dob

    # ---- backward of the chunked prefill (fp32, then bf16 I/O) ------------------
    if want("prefill_bwd"):
        wb = synth.WORKLOADS["prefill_bwd_8k"]
        xb = synth.prefill_inputs(wb.B, wb.T, wb.H, torch.float32, seed=wb.seed,
                                  g_shift=wb.g_shift, h0_std=wb.h0_std, device=dev)
        gbn = torch.Generator(device=dev).manual_seed(wb.seed + 1)
        xb["dout"] = torch.randn((wb.B, wb.T, wb.H, 128), generator=gbn, device=dev)
        xb["dhT"] = 0.1 * torch.randn((wb.B, wb.H, 128, 128), generator=gbn, device=dev)

        def prefill_bwd():
            libkda.chunk_bwd(xb["q"], xb["k"], xb["v"], xb["g"], xb["beta"], xb["scale"],
                             xb["dout"], h0=xb["h0"], dhT=xb["dhT"])

        nsteps = max(3, args.steps // 4)
        t = time_op(torch, prefill_bwd, nsteps, args.warmup)
        pb_chunks = wb.B * wb.H * ((wb.T + 63) // 64)
        pb_flop = pb_chunks * BWD_CHUNK_FLOP_PER_CHUNK_HEAD
        tf = pb_flop / (t[0] / 1e3) / 1e12
        nb = wb.B * wb.T * wb.H * BWD_CHUNK_BYTES_PER_TOKEN_HEAD + 3 * wb.B * wb.H * STATE_BYTES
        print(f"# prefill backward (fp32): {t[0]:.3f} ms/call, {tf:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        res["prefill_bwd"] = {
            "workload": f"prefill_bwd_8k: backward of one fp32 KDA layer prefill, B={wb.B} "
                        f"H={wb.H} T={wb.T} d=128, h0 and dhT ~ N(0, 0.1^2), dout ~ N(0, 1) "
                        "(kda_chunk_bwd_f32: gradients of q, k, v, g, beta and h0)",
            **times(*t), "Mtok_s": round(wb.B * wb.T / (t[0] / 1e3) / 1e6, 3),
            "roofline": {
                "bound": "alu",
                "kernel": "kda_chunk_bwd_f32 (prep, two state scans, chunk gradients; one call)",
                "achieved": round(tf, 2), "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / FP32_VALU_PEAK_TFLOPS, 4), "algorithmic_flop_per_call": pb_flop,
                "traffic": measured_traffic("prefill_bwd_8k"), "algorithmic_bytes_per_call": nb,
                "hbm_GBps_algorithmic": round(nb / (t[0] / 1e3) / 1e9, 1),
                "note": "algorithmic fp32 flops against the fp32 matrix peak; the scans' and "
                        "the chunk kernel's [64][128] products run as three bf16 products of "
                        "hi / lo pairs each (fp32-like accuracy), the rest on fp32 matrix cores"}}
        for key in ("q", "k", "v", "dout"):
            xb[key] = xb[key].to(torch.bfloat16)
        t = time_op(torch, prefill_bwd, nsteps, args.warmup)
        tf = pb_flop / (t[0] / 1e3) / 1e12
        nb = wb.B * wb.T * wb.H * BWD_CHUNK_BF16_BYTES_PER_TOKEN_HEAD + \
            3 * wb.B * wb.H * STATE_BYTES
        print(f"# prefill backward (bf16 I/O): {t[0]:.3f} ms/call, {tf:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        res["prefill_bwd_bf16"] = {
            "workload": "prefill_bwd_8k with bf16 q, k, v, dout in and bf16 dq, dk, dv out "
                        "(kda_chunk_bwd), fp32 arithmetic",
            **times(*t), "Mtok_s": round(wb.B * wb.T / (t[0] / 1e3) / 1e6, 3),
            "roofline": {"bound": "alu", "achieved": round(tf, 2), "peak": FP32_VALU_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / FP32_VALU_PEAK_TFLOPS, 4),
                         "algorithmic_flop_per_call": pb_flop, "algorithmic_bytes_per_call": nb}}
        del xb

    # ---- the small fp32 case through both paths (latency) ---------------------
    if want("small_f32"):
        ws_ = synth.WORKLOADS["small_f32"]
        xs_ = synth.workload_inputs(ws_, dev)
        o_s = torch.empty_like(xs_["v"])
        h_s = torch.empty((ws_.B, ws_.H, 128, 128), device=dev)

        def small_chunk():
            libkda.chunk_fwd(xs_["q"], xs_["k"], xs_["v"], xs_["g"], xs_["beta"], xs_["scale"],
                             None, out=o_s, hT=h_s)

        tc = time_op(torch, small_chunk, 50, args.warmup)
        steps_s = [{kk: xs_[kk][:, t].contiguous() for kk in ("q", "k", "v", "g", "beta")}
                   for t in range(ws_.T)]
        S_s = torch.zeros((ws_.B, ws_.H, 128, 128), device=dev)
        o_r = torch.empty((ws_.B, ws_.H, 128), device=dev)

        def small_recurrent():  # the whole sequence: 256 decode steps
            S_s.zero_()
            for x in steps_s:
                libkda.recurrent_step(x["q"], x["k"], x["v"], x["g"], x["beta"], xs_["scale"],
                                      S_s, out=o_r)

        tr = time_op(torch, small_recurrent, 5, 1)
        t_or = None if args.no_cpu_baseline else oracle_sample(xs_, range(ws_.H), ws_.T)
        print(f"# small fp32 (B=1 H=2 T=256): chunked {tc[0] * 1e3:.1f} us/call, recurrent "
              f"{tr[0] * 1e3:.1f} us for 256 steps ({tr[0] * 1e3 / ws_.T:.2f} us/step)",
              file=sys.stderr, flush=True)
        res["small_f32"] = {
            "workload": "small_f32: B=1 H=2 T=256 d=128, fp32 q/k/v/o, zero initial state, "
                        "seed 0",
            "chunked_us_per_call": round(tc[0] * 1e3, 2),
            "chunked_us_median": round(tc[1] * 1e3, 2),
            "chunked_us_min": round(tc[2] * 1e3, 2),
            "recurrent_us_for_256_steps": round(tr[0] * 1e3, 2),
            "recurrent_us_per_step": round(tr[0] * 1e3 / ws_.T, 3),
            "note": "latency-bound (1.44 MB of algorithmic bytes, 0.18 us at 8 TB/s); the "
                    "chunked path is one kda_chunk_fwd_f32, the recurrent path 256 "
                    "kda_recurrent_step_f32 calls launched from Python",
            "cpu_baseline": None if t_or is None else {
                "us": round(t_or * 1e6, 1), "kind": "oracle", "sample": "the whole workload"}}
        del xs_, o_s, h_s, steps_s, S_s, o_r

    # ---- one 96-head layer at T = 4096 ------------------------------------------
    if want("layer_4k"):
        wl = synth.WORKLOADS["layer_4k"]
        xl = synth.workload_inputs(wl, dev)
        o_l = torch.empty_like(xl["v"])
        h_l = torch.empty((wl.B, wl.H, 128, 128), device=dev)

        def layer():
            libkda.chunk_fwd(xl["q"], xl["k"], xl["v"], xl["g"], xl["beta"], xl["scale"], None,
                             out=o_l, hT=h_l)

        t = time_op(torch, layer, args.steps, args.warmup)
        nb = wl.B * wl.T * wl.H * PREFILL_BYTES_PER_TOKEN_HEAD + wl.B * wl.H * STATE_BYTES
        gb = nb / (t[0] / 1e3) / 1e9
        t_ol = None if args.no_cpu_baseline else oracle_sample(xl, range(wl.H), wl.T)
        print(f"# layer_4k: {t[0]:.3f} ms/call, {wl.B * wl.T / (t[0] / 1e3) / 1e6:.2f} Mtok/s, "
              f"{gb:.0f} GB/s", file=sys.stderr, flush=True)
        res["layer_4k"] = {
            "workload": "layer_4k: B=1 H=96 T=4096 d=128, bf16 q/k/v, fp32 g/beta, zero "
                        "initial state (no h0 read), seed 1",
            **times(*t), "Mtok_s": round(wl.B * wl.T / (t[0] / 1e3) / 1e6, 3),
            "roofline": hbm(gb, nb),
            "cpu_baseline": None if t_ol is None else {
                "value": round(wl.B * wl.T / t_ol / 1e6, 5), "unit": "Mtok/s", "kind": "oracle",
                "sample": f"the whole workload, {t_ol:.2f} s of oracle time"}}
        del xl, o_l, h_l

    # ---- the million-token prefill ----------------------------------------------
    if want("prefill_1m"):
        torch.cuda.empty_cache()
        wm = synth.WORKLOADS["prefill_1m"]
        xm = synth.workload_inputs(wm, dev)
        o_m = torch.empty_like(xm["v"])
        h_m = torch.empty((wm.B, wm.H, 128, 128), device=dev)

        def prefill_1m():
            libkda.chunk_fwd(xm["q"], xm["k"], xm["v"], xm["g"], xm["beta"], xm["scale"], None,
                             out=o_m, hT=h_m)

        t = time_op(torch, prefill_1m, max(2, args.steps // 5), 1)
        nb = wm.B * wm.T * wm.H * PREFILL_BYTES_PER_TOKEN_HEAD + wm.B * wm.H * STATE_BYTES
        gb = nb / (t[0] / 1e3) / 1e9
        m_heads, m_tokens = range(0, wm.H, wm.H // 16), 32768
        t_om = None if args.no_cpu_baseline else oracle_sample(xm, m_heads, m_tokens)
        print(f"# prefill_1m: {t[0]:.2f} ms/call, {wm.B * wm.T / (t[0] / 1e3) / 1e6:.2f} Mtok/s, "
              f"{gb:.0f} GB/s", file=sys.stderr, flush=True)
        res["prefill_1m"] = {
            "workload": "prefill_1m: B=1 H=96 T=1048576 d=128, bf16 q/k/v, fp32 g = -5 "
                        "sigmoid(x - 6) and beta, zero initial state (no h0 read), seed 4 "
                        "(155 GB resident)",
            **times(*t, nd=3), "Mtok_s": round(wm.B * wm.T / (t[0] / 1e3) / 1e6, 3),
            "roofline": hbm(gb, nb),
            "cpu_baseline": None if t_om is None else {
                "value": round(len(m_heads) * m_tokens / wm.H / t_om / 1e6, 6),
                "unit": "Mtok/s", "kind": "oracle",
                "sample": f"heads {list(m_heads)} x the first {m_tokens} tokens ({t_om:.2f} s "
                          "of oracle time), scaled to all 96 heads: Mtok/s = sampled "
                          "token-heads / 96 / seconds"}}
        del xm, o_m, h_m
        torch.cuda.empty_cache()

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, min(args.cpu_sample_tokens, w.T))
        print(f"# cpu oracle: {cpu['value']:.5f} Mtok/s on {cpu['cores']} threads",
              file=sys.stderr, flush=True)

    line = {
        "metric": "KDA chunk-fwd Mtok/s at H=96,T=64K; decode state GB/s; % of roofline",
        "value": round(mtok, 3),
        "unit": "Mtok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(ms_med, 4),
        "ms_per_step_min": round(ms_min, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "prefill_64k: one KDA layer, B=1 H=96 T=65536 d=128, bf16 q/k/v, "
                        "fp32 g/beta, fp32 state, h0 ~ N(0, 0.1^2), seed 2",
            "B": w.B, "H": w.H, "T": w.T, "head_dim": 128, "chunk": 64,
            "parallelism": "single GPU",
        },
        "roofline": hbm(pre_gbps, pre_bytes,
                        kernel="kda_chunk_fwd (kda_prep16_kernel + kda_scan16_kernel, one call)",
                        traffic=measured_traffic("prefill_64k")),
        "mfma": {
            "algorithmic_flop_per_call": token_heads * PREFILL_FLOP_PER_TOKEN_HEAD,
            "achieved_TFLOPs": round(pre_tflops, 1),
            "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
            "frac": round(pre_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "note": "algorithmic flops at a fixed 64-token chunk; the binding roofline is HBM",
        },
    }
    for key in ("prefill_g16", "prefill_conv", "decode_conv", "decode_bwd", "prefill_bwd",
                "prefill_bwd_bf16", "decode", "small_f32", "layer_4k", "prefill_1m"):
        line[key] = res.get(key)
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
