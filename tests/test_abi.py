"""The C-ABI boundary, on the CPU: the library loads, exports every entry
point ``include/kda.h`` declares, and rejects bad arguments with the
documented status codes before making any HIP call (so no GPU is needed)."""
import ctypes
import math
import os
import re

import pytest

from linear_attention_07_amd import build as kbuild
from linear_attention_07_amd import libkda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    # The validation tests below hand the library fake device addresses; on a
    # host with a GPU a call that slipped past validation would launch on
    # them, so they run on GPU-less hosts only.
    import torch
    if torch.cuda.is_available():
        pytest.skip("argument validation is exercised on hosts without a GPU")
    if not os.path.exists(libkda.LIB_PATH):
        kbuild.build()
    return libkda.load()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"KDA_API\s+[\w\s\*]*?\b(kda_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_symbols() == sorted(libkda.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    names = ("KDA_OK", "KDA_ERR_INVALID_ARG", "KDA_ERR_UNSUPPORTED", "KDA_ERR_HIP",
             "KDA_ERR_NO_MEMORY", "KDA_ERR_PRECONDITION", "KDA_ERR_DEVICE")
    header = open(HEADER).read()
    for code, name in enumerate(names):
        s = libkda.status_string(code)
        assert s.startswith(name + ":"), (code, s)
        assert re.search(rf"\b{name}\s*=\s*{code}\b", header), name   # the header's value
        assert getattr(libkda, name) == code
    assert "unknown" in libkda.status_string(99)


def test_trim_without_pools_is_a_no_op(lib):
    # no pool was ever created on this GPU-less host: nothing to hand back
    assert lib.kda_trim_workspace() == libkda.KDA_OK


# Fake but 16-byte aligned, non-null device addresses: validation must fail
# (or succeed as a no-op) before anything dereferences them.
A = 1 << 20
P = [ctypes.c_void_p(A * (i + 1)) for i in range(12)]
NULL = None


def chunk(lib, fn="kda_chunk_fwd", q=P[0], k=P[1], v=P[2], g=P[3], beta=P[4], scale=1.0,
          h0=NULL, out=P[5], hT=NULL, B=1, T=4, H=1):
    return getattr(lib, fn)(q, k, v, g, beta, scale, h0, out, hT, B, T, H, None)


def step(lib, fn="kda_recurrent_step", q=P[0], k=P[1], v=P[2], g=P[3], beta=P[4], scale=1.0,
         S=P[6], out=P[5], B=1, H=1):
    return getattr(lib, fn)(q, k, v, g, beta, scale, S, out, B, H, None)


@pytest.mark.parametrize("fn", ["kda_chunk_fwd", "kda_chunk_fwd_f32", "kda_chunk_fwd_g16"])
def test_chunk_invalid_arguments(lib, fn):
    INV = libkda.KDA_ERR_INVALID_ARG
    assert chunk(lib, fn, B=-1) == INV
    assert chunk(lib, fn, T=-1) == INV
    assert chunk(lib, fn, H=-3) == INV
    assert chunk(lib, fn, scale=math.inf) == INV
    assert chunk(lib, fn, scale=math.nan) == INV
    for name in ("q", "k", "v", "g", "beta", "out"):
        assert chunk(lib, fn, **{name: NULL}) == INV, name
    for name in ("q", "k", "v", "g", "out"):
        assert chunk(lib, fn, **{name: ctypes.c_void_p(A + 8)}) == INV, name
    assert chunk(lib, fn, beta=ctypes.c_void_p(A * 5 + 2)) == INV
    assert chunk(lib, fn, h0=ctypes.c_void_p(A * 7 + 4)) == INV
    # out overlapping an input
    assert chunk(lib, fn, out=ctypes.c_void_p(A + 256)) == INV
    # partially overlapping h0 / hT
    assert chunk(lib, fn, h0=P[7], hT=ctypes.c_void_p(A * 8 + 4096)) == INV


@pytest.mark.parametrize("fn", ["kda_chunk_fwd", "kda_chunk_fwd_f32", "kda_chunk_fwd_g16"])
def test_chunk_empty_is_a_no_op(lib, fn):
    assert chunk(lib, fn, B=0) == libkda.KDA_OK
    assert chunk(lib, fn, H=0) == libkda.KDA_OK
    # T == 0 without a final-state buffer: nothing to do, pointers unused
    assert chunk(lib, fn, T=0, q=NULL, k=NULL, v=NULL, g=NULL, beta=NULL, out=NULL) == libkda.KDA_OK
    # T == 0 with hT == h0: the state is already in place
    assert chunk(lib, fn, T=0, h0=P[7], hT=P[7]) == libkda.KDA_OK


@pytest.mark.parametrize("fn", ["kda_chunk_fwd", "kda_chunk_fwd_f32", "kda_chunk_fwd_g16"])
def test_chunk_refuses_more_scan_workgroups_than_a_launch_takes(lib, fn):
    # two value slices per head: past 2^23 scan workgroups the call is refused
    # before any HIP call (buffers far apart, so no overlap check trips first)
    far = [ctypes.c_void_p((i + 1) << 44) for i in range(6)]
    H = (1 << 22) + 1
    assert chunk(lib, fn, q=far[0], k=far[1], v=far[2], g=far[3], beta=far[4], out=far[5],
                 H=H) == libkda.KDA_ERR_UNSUPPORTED


def conv(lib, q=P[0], k=P[1], v=P[2], wq=P[8], wk=P[9], wv=P[10], conv_in=NULL, conv_out=NULL,
         g=P[3], beta=P[4], scale=1.0, h0=NULL, gate=NULL, out=P[5], hT=NULL, B=1, T=4, H=1):
    return lib.kda_chunk_fwd_conv(q, k, v, wq, wk, wv, conv_in, conv_out, g, beta, scale, h0, gate,
                                  out, hT, B, T, H, None)


def test_conv_invalid_arguments(lib):
    INV = libkda.KDA_ERR_INVALID_ARG
    assert conv(lib, B=-1) == INV
    assert conv(lib, scale=math.nan) == INV
    for name in ("q", "k", "v", "g", "beta", "out", "wq", "wk", "wv"):
        assert conv(lib, **{name: NULL}) == INV, name
    for name in ("wq", "wk", "wv", "conv_in", "conv_out"):
        assert conv(lib, **{name: ctypes.c_void_p(A * 12 + 8)}) == INV, name
    # conv_in and conv_out partly overlapping (equal is the in-place update)
    assert conv(lib, conv_in=P[11], conv_out=ctypes.c_void_p(A * 12 + 512)) == INV
    # out over a weight or a conv buffer; conv_out over a weight or an input
    assert conv(lib, out=ctypes.c_void_p(A * 9 + 256)) == INV
    assert conv(lib, conv_in=P[11], out=ctypes.c_void_p(A * 12 + 1024)) == INV
    assert conv(lib, conv_out=ctypes.c_void_p(A * 10 + 1024)) == INV
    assert conv(lib, conv_out=ctypes.c_void_p(A * 2 + 512)) == INV
    # the gate: misaligned, under out, under conv_out
    assert conv(lib, gate=ctypes.c_void_p(A * 12 + 8)) == INV
    assert conv(lib, gate=ctypes.c_void_p(A * 6 - 256)) == INV
    assert conv(lib, conv_out=P[11], gate=ctypes.c_void_p(A * 12 + 256)) == INV


def test_conv_empty_is_a_no_op(lib):
    assert conv(lib, B=0) == libkda.KDA_OK
    assert conv(lib, H=0) == libkda.KDA_OK
    # no tokens, no state to produce
    assert conv(lib, T=0, q=NULL, k=NULL, v=NULL, g=NULL, beta=NULL, out=NULL) == libkda.KDA_OK
    # no tokens, conv state updated in place: already there
    assert conv(lib, T=0, conv_in=P[11], conv_out=P[11], h0=P[7], hT=P[7]) == libkda.KDA_OK


@pytest.mark.parametrize("fn", ["kda_recurrent_step", "kda_recurrent_step_f32"])
def test_step_invalid_arguments(lib, fn):
    INV = libkda.KDA_ERR_INVALID_ARG
    assert step(lib, fn, B=-1) == INV
    assert step(lib, fn, H=-1) == INV
    assert step(lib, fn, scale=-math.inf) == INV
    for name in ("q", "k", "v", "g", "beta", "S", "out"):
        assert step(lib, fn, **{name: NULL}) == INV, name
    for name in ("q", "k", "v", "g", "S", "out"):
        assert step(lib, fn, **{name: ctypes.c_void_p(A * 9 + 8)}) == INV, name
    # state overlapping out, out overlapping v
    assert step(lib, fn, out=ctypes.c_void_p(A * 7 + 64)) == INV
    assert step(lib, fn, out=ctypes.c_void_p(A * 3 + 16)) == INV
    assert step(lib, fn, B=0) == libkda.KDA_OK
    assert step(lib, fn, H=0) == libkda.KDA_OK


def step_conv(lib, q=P[0], k=P[1], v=P[2], wq=P[8], wk=P[9], wv=P[10], cs=P[11], g=P[3],
              beta=P[4], scale=1.0, S=P[6], gate=NULL, out=P[5], B=1, H=1):
    return lib.kda_recurrent_step_conv(q, k, v, wq, wk, wv, cs, g, beta, scale, S, gate, out, B,
                                       H, None)


def test_step_conv_invalid_arguments(lib):
    INV = libkda.KDA_ERR_INVALID_ARG
    assert step_conv(lib, B=-1) == INV
    assert step_conv(lib, scale=math.nan) == INV
    for name in ("q", "k", "v", "wq", "wk", "wv", "cs", "g", "beta", "S", "out"):
        assert step_conv(lib, **{name: NULL}) == INV, name
    for name in ("wq", "wk", "wv", "cs"):
        assert step_conv(lib, **{name: ctypes.c_void_p(A * 12 + 8)}) == INV, name
    # the conv state over an input, a tap, the attention state or out
    assert step_conv(lib, cs=ctypes.c_void_p(A * 1 + 128)) == INV
    assert step_conv(lib, cs=ctypes.c_void_p(A * 9 + 16)) == INV
    assert step_conv(lib, cs=ctypes.c_void_p(A * 7 + 1024)) == INV
    assert step_conv(lib, cs=ctypes.c_void_p(A * 6 - 256)) == INV
    # out over a tap; the gate misaligned or under out / the conv state
    assert step_conv(lib, out=ctypes.c_void_p(A * 10 + 256)) == INV
    assert step_conv(lib, gate=ctypes.c_void_p(A * 12 + 8)) == INV
    assert step_conv(lib, gate=ctypes.c_void_p(A * 6 - 128)) == INV
    assert step_conv(lib, gate=ctypes.c_void_p(A * 12 + 512)) == INV
    assert step_conv(lib, B=0) == libkda.KDA_OK
    assert step_conv(lib, H=0) == libkda.KDA_OK


def step_bwd(lib, fn="kda_recurrent_step_bwd_f32", **kw):
    args = dict(q=P[0], k=P[1], v=P[2], g=P[3], beta=P[4], scale=1.0, S_prev=P[5], dout=P[6],
                dS=P[7], dq=P[8], dk=P[9], dv=P[10], dg=P[11], dbeta=ctypes.c_void_p(A * 13),
                B=1, H=1)
    args.update(kw)
    return getattr(lib, fn)(*args.values(), None)


@pytest.mark.parametrize("fn", ["kda_recurrent_step_bwd_f32", "kda_recurrent_step_bwd"])
def test_step_bwd_invalid_arguments(lib, fn):
    INV = libkda.KDA_ERR_INVALID_ARG
    assert step_bwd(lib, fn, B=-1) == INV
    assert step_bwd(lib, fn, scale=math.inf) == INV
    for name in ("q", "k", "v", "g", "beta", "S_prev", "dout", "dS", "dq", "dk", "dv", "dg",
                 "dbeta"):
        assert step_bwd(lib, fn, **{name: NULL}) == INV, name
    for name in ("q", "dS", "dq", "dg"):
        assert step_bwd(lib, fn, **{name: ctypes.c_void_p(A * 20 + 8)}) == INV, name
    # a written buffer over an input, over the state, over another output
    # (offsets inside the smaller, bf16 vectors of 256 bytes as well)
    assert step_bwd(lib, fn, dq=ctypes.c_void_p(A * 1 + 128)) == INV
    assert step_bwd(lib, fn, dS=ctypes.c_void_p(A * 6 - 4096)) == INV
    assert step_bwd(lib, fn, dv=ctypes.c_void_p(A * 9 + 128)) == INV
    assert step_bwd(lib, fn, dbeta=ctypes.c_void_p(A * 12 + 64)) == INV
    assert step_bwd(lib, fn, B=0) == libkda.KDA_OK
    assert step_bwd(lib, fn, H=0) == libkda.KDA_OK


def test_binding_rejects_bad_tensors():
    import torch
    q = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        libkda.chunk_fwd(q, q, q, q.float(), torch.zeros(1, 4, 1), 1.0)  # CPU tensors
    with pytest.raises(ValueError):
        libkda.chunk_fwd(q[..., :64], q, q, q.float(), torch.zeros(1, 4, 1), 1.0)
    w = torch.zeros(1, 128, 4)
    with pytest.raises(ValueError):
        libkda.chunk_fwd_conv(q, q, q, w, w, w, q.float(), torch.zeros(1, 4, 1), 1.0)
    with pytest.raises(ValueError):
        libkda.recurrent_step(q[0], q[0], q[0], q[0].float(), torch.zeros(4, 1),
                              1.0, torch.zeros(4, 1, 128, 128))
    with pytest.raises(ValueError):
        libkda.recurrent_step_conv(q[0], q[0], q[0], w, w, w,
                                   torch.zeros(3, 4, 3, 1, 128, dtype=torch.bfloat16),
                                   q[0].float(), torch.zeros(4, 1), 1.0,
                                   torch.zeros(4, 1, 128, 128))


def test_oracle_is_not_reachable_from_the_product():
    """The library and its binding never load the test oracle."""
    pkg = os.path.join(ROOT, "linear_attention_07_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, re.M), f
                assert "_kda_oracle" not in text and "kda_oracle_run" not in text, f


# Fake addresses for the prefill backward: 15 buffers, 1 MiB apart (or 1 TiB
# apart for sizes that would otherwise overlap).
def chunk_bwd(lib, spacing=A, **kw):
    names = ("q", "k", "v", "g", "beta", "h0", "dout", "dhT", "dq", "dk", "dv", "dg", "dbeta",
             "dh0")
    args = {n: ctypes.c_void_p(spacing * (i + 1)) for i, n in enumerate(names)}
    args.update(scale=1.0, B=1, T=4, H=1)
    args.update(kw)
    return lib.kda_chunk_bwd_f32(
        args["q"], args["k"], args["v"], args["g"], args["beta"], args["scale"], args["h0"],
        args["dout"], args["dhT"], args["dq"], args["dk"], args["dv"], args["dg"], args["dbeta"],
        args["dh0"], args["B"], args["T"], args["H"], None)


def test_chunk_bwd_invalid_arguments(lib):
    INV = libkda.KDA_ERR_INVALID_ARG
    for bad in (dict(B=-1), dict(T=-1), dict(H=-1), dict(scale=math.inf), dict(scale=math.nan)):
        assert chunk_bwd(lib, **bad) == INV, bad
    for name in ("q", "k", "v", "g", "beta", "dout", "dq", "dk", "dv", "dg", "dbeta"):
        assert chunk_bwd(lib, **{name: NULL}) == INV, name
    for name in ("q", "g", "dout", "h0", "dhT", "dq", "dg", "dh0"):
        assert chunk_bwd(lib, **{name: ctypes.c_void_p(A * 20 + 8)}) == INV, name
    for name in ("beta", "dbeta"):
        assert chunk_bwd(lib, **{name: ctypes.c_void_p(A * 20 + 2)}) == INV, name
    # a written buffer over an input, over the states, over another output
    assert chunk_bwd(lib, dq=ctypes.c_void_p(A * 2 + 128)) == INV       # over k
    assert chunk_bwd(lib, dg=ctypes.c_void_p(A * 7 + 1024)) == INV      # over dout
    assert chunk_bwd(lib, dv=ctypes.c_void_p(A * 12 - 1024)) == INV     # over dg
    assert chunk_bwd(lib, dbeta=ctypes.c_void_p(A * 5 + 8)) == INV      # over beta
    assert chunk_bwd(lib, dh0=ctypes.c_void_p(A * 6 + 4096)) == INV     # over h0
    assert chunk_bwd(lib, dh0=ctypes.c_void_p(A * 8 - 4096)) == INV     # over dhT
    assert chunk_bwd(lib, dk=ctypes.c_void_p(A * 14 + 512)) == INV      # over dh0
    # no batch or no heads: nothing to do
    assert chunk_bwd(lib, B=0) == libkda.KDA_OK
    assert chunk_bwd(lib, H=0) == libkda.KDA_OK
    # no tokens and no initial-state gradient asked for: nothing to do
    assert chunk_bwd(lib, T=0, dh0=NULL) == libkda.KDA_OK


def test_chunk_bwd_segments_any_length(lib):
    # 4096 heads x 2049 chunks of workgroups would exceed the launch limit in
    # one segment; the call is split into segments instead, so validation
    # passes it on to the device (the first HIP call fails on this host)
    assert chunk_bwd(lib, spacing=1 << 40, H=4096, T=64 * 2048 + 1) == libkda.KDA_ERR_HIP
    # a head count past the scan's grid is still refused before any HIP call
    assert chunk_bwd(lib, spacing=1 << 46, B=2, H=(1 << 21) + 1, T=64) == \
        libkda.KDA_ERR_UNSUPPORTED


def test_chunk_bwd_bf16_invalid_arguments(lib):
    INV = libkda.KDA_ERR_INVALID_ARG
    # the bf16 entry point shares the validation; the bf16 arrays are half the size
    def call(**kw):
        names = ("q", "k", "v", "g", "beta", "h0", "dout", "dhT", "dq", "dk", "dv", "dg",
                 "dbeta", "dh0")
        args = {n: ctypes.c_void_p(A * (i + 1)) for i, n in enumerate(names)}
        args.update(scale=1.0, B=1, T=4, H=1)
        args.update(kw)
        return lib.kda_chunk_bwd(
            args["q"], args["k"], args["v"], args["g"], args["beta"], args["scale"],
            args["h0"], args["dout"], args["dhT"], args["dq"], args["dk"], args["dv"],
            args["dg"], args["dbeta"], args["dh0"], args["B"], args["T"], args["H"], None)
    assert call(B=-1) == INV
    assert call(q=NULL) == INV
    assert call(dv=ctypes.c_void_p(A * 20 + 8)) == INV
    assert call(dq=ctypes.c_void_p(A * 2 + 512)) == INV     # inside k's 1 KiB of bf16
    assert call(dg=ctypes.c_void_p(A * 4 + 1024)) == INV    # inside g's 2 KiB of fp32
    assert call(B=0) == libkda.KDA_OK
    assert call(T=0, dh0=NULL) == libkda.KDA_OK


@pytest.mark.parametrize("fn", ["kda_chunk_bwd_f32", "kda_chunk_bwd"])
@pytest.mark.parametrize("pair", [("dq", "dk"), ("dv", "dout"), ("dq", "q"), ("dg", "g"),
                                  ("dbeta", "beta"), ("dh0", "dhT"), ("dh0", "h0")])
def test_chunk_bwd_rejects_a_buffer_passed_twice(lib, fn, pair):
    """A written buffer given at the very address of another argument is an
    overlap like any other (kda.h: every written buffer overlaps no other
    argument)."""
    names = ("q", "k", "v", "g", "beta", "h0", "dout", "dhT", "dq", "dk", "dv", "dg", "dbeta",
             "dh0")
    args = {n: ctypes.c_void_p(A * (i + 1)) for i, n in enumerate(names)}
    args[pair[0]] = args[pair[1]]
    rc = getattr(lib, fn)(
        args["q"], args["k"], args["v"], args["g"], args["beta"], 1.0, args["h0"], args["dout"],
        args["dhT"], args["dq"], args["dk"], args["dv"], args["dg"], args["dbeta"], args["dh0"],
        1, 4, 1, None)
    assert rc == libkda.KDA_ERR_INVALID_ARG, pair


def test_noalloc_validation_and_size_limit(lib):
    """kda_chunk_fwd_noalloc validates like kda_chunk_fwd, and refuses, before
    any HIP call, a B * H whose chunk records and carried state do not fit its
    64 MiB scratch (one chunk record and one state per head)."""
    INV = libkda.KDA_ERR_INVALID_ARG
    for bad in (dict(B=-1), dict(scale=math.nan), dict(q=NULL), dict(out=P[0]),
                dict(g=ctypes.c_void_p(A * 20 + 8))):
        assert chunk(lib, fn="kda_chunk_fwd_noalloc", **bad) == INV, bad
    assert chunk(lib, fn="kda_chunk_fwd_noalloc", B=0) == libkda.KDA_OK
    big = dict(fn="kda_chunk_fwd_noalloc", T=640, H=1024)
    sp = [ctypes.c_void_p((i + 1) << 36) for i in range(6)]
    assert chunk(lib, q=sp[0], k=sp[1], v=sp[2], g=sp[3], beta=sp[4], out=sp[5], **big) == \
        libkda.KDA_ERR_UNSUPPORTED
