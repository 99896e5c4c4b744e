"""The C ABI of libparallax on the host: symbols, split planning, validation.

No call here reaches a kernel launch: every call either is host-only
(status strings, split planning, workspace sizing) or fails argument
validation, which the library performs before any HIP call.
"""

import ctypes
import os
import re

import pytest

import transformer_attention_parallax_amd as px

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "parallax.h")

FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"PARALLAX_API[^;(]*?\b(parallax_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return px.library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("parallax_decode", "parallax_fwd", "parallax_decode_workspace_size",
              "parallax_fwd_workspace_size", "parallax_decode_splits",
              "parallax_status_string", "parallax_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"
        assert name in px.SIGNATURES, f"{name} has no binding signature"


def test_exports_nothing_else():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", px.LIBRARY],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    ours = {s for s in exported if s.startswith("parallax_")}
    assert ours == set(declared_functions())


def test_status_strings(lib):
    for code in range(5):
        s = lib.parallax_status_string(code)
        assert s and s != b"unknown status"
    assert lib.parallax_status_string(99) == b"unknown status"


def test_split_planning():
    # plenty of (b, h) streams: one split, no workspace
    assert px.decode_splits(256, 16, 128, 8192) == 1
    assert px.decode_workspace_size(256, 16, 128, 8192) == 0
    # few streams: split the keys, every split at least 256 keys; contexts
    # under 1024 keys stay whole
    s = px.decode_splits(1, 16, 128, 4096)
    assert 1 < s <= 4096 // 256
    assert px.decode_splits(1, 16, 128, 2048) == 8
    assert px.decode_splits(1, 16, 128, 1023) == 1
    # one record per (b, h, split)
    assert px.decode_workspace_size(1, 16, 128, 4096) == 16 * s * (4 + 256) * 4
    assert px.decode_workspace_size(3, 30, 64, 4096, 2) == 90 * 2 * (4 + 128) * 4
    # explicit requests are honoured, clamped to 64-key granularity
    assert px.decode_splits(1, 1, 128, 4096, num_splits=7) == 7
    assert px.decode_splits(1, 1, 128, 100, num_splits=50) == 2
    assert px.decode_splits(1, 1, 64, 1, num_splits=3) == 1
    assert px.decode_splits(1, 1, 128, 0) == 1
    # short contexts never split automatically
    assert px.decode_splits(1, 16, 128, 128) == 1


def test_split_planning_covers_the_context():
    for L in (1, 63, 64, 65, 1000, 4096, 32768):
        for req in (0, 1, 2, 3, 7, 64, 1000):
            s = px.decode_splits(1, 16, 128, L, num_splits=req)
            assert 1 <= s <= max(1, -(-L // 64))


def _decode(lib, **kw):
    a = dict(q=FAKE, q_sb=16 * 128, q_sh=128, rho=FAKE, r_sb=16 * 128, r_sh=128,
             k=FAKE, v=FAKE, kv_sb=16 * 4096 * 128, kv_sh=4096 * 128, kv_sl=128,
             seqlens=None, out=FAKE, o_sb=16 * 128, o_sh=128, B=1, H=16, D=128,
             L=4096, scale=0.088, idt=px.BF16, odt=px.F32, ns=0, ws=None,
             wsb=0, stream=None)
    a.update(kw)
    return lib.parallax_decode(
        a["q"], a["q_sb"], a["q_sh"], a["rho"], a["r_sb"], a["r_sh"], a["k"],
        a["v"], a["kv_sb"], a["kv_sh"], a["kv_sl"], a["seqlens"], a["out"],
        a["o_sb"], a["o_sh"], a["B"], a["H"], a["D"], a["L"], a["scale"],
        a["idt"], a["odt"], a["ns"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), px.ERR_INVALID_ARG),
    # rho NULL is plain softmax attention: validation goes on (and stops at
    # the missing workspace of this split decode)
    (dict(rho=None), px.ERR_WORKSPACE),
    (dict(k=None), px.ERR_INVALID_ARG),
    (dict(out=None), px.ERR_INVALID_ARG),
    (dict(D=96), px.ERR_UNSUPPORTED),
    (dict(D=0), px.ERR_INVALID_ARG),
    (dict(B=-1), px.ERR_INVALID_ARG),
    (dict(L=-5), px.ERR_INVALID_ARG),
    (dict(idt=7), px.ERR_INVALID_ARG),
    (dict(odt=-1), px.ERR_INVALID_ARG),
    (dict(scale=float("nan")), px.ERR_INVALID_ARG),
    (dict(scale=float("inf")), px.ERR_INVALID_ARG),
    (dict(q=FAKE + 2), px.ERR_UNSUPPORTED),
    (dict(k=FAKE + 8), px.ERR_UNSUPPORTED),
    (dict(kv_sl=129), px.ERR_UNSUPPORTED),
    (dict(q_sh=-128), px.ERR_INVALID_ARG),
    (dict(out=FAKE + 2), px.ERR_UNSUPPORTED),
    (dict(seqlens=FAKE + 2), px.ERR_UNSUPPORTED),
    (dict(ns=-1), px.ERR_INVALID_ARG),
    # 16 streams of 4096 keys need splits, hence a workspace
    (dict(ws=None, wsb=0), px.ERR_WORKSPACE),
    (dict(ws=FAKE, wsb=100), px.ERR_WORKSPACE),
    (dict(ws=FAKE + 4, wsb=1 << 30), px.ERR_UNSUPPORTED),
])
def test_decode_validation(lib, kw, status):
    assert _decode(lib, **kw) == status
    assert lib.parallax_last_error() != b""


def test_decode_empty_problem_is_ok(lib):
    assert _decode(lib, B=0, q=None, k=None, v=None, out=None) == px.OK
    assert _decode(lib, H=0) == px.OK


def _fwd(lib, **kw):
    s = (4096 * 16 * 128, 16 * 128, 128)
    a = dict(q=FAKE, k=FAKE, v=FAKE, rho=FAKE, out=FAKE, qs=s, ks=s, vs=s,
             rs=s, os=s, B=8, N=4096, H=16, D=128, scale=0.088, causal=1,
             idt=px.BF16, odt=px.F32, ws=FAKE, wsb=8 * 16 * 4096 * 128 * 2,
             stream=None)
    a.update(kw)
    return lib.parallax_fwd(
        a["q"], *a["qs"], a["k"], *a["ks"], a["v"], *a["vs"], a["rho"],
        *a["rs"], a["out"], *a["os"], a["B"], a["N"], a["H"], a["D"],
        a["scale"], a["causal"], a["idt"], a["odt"], a["ws"], a["wsb"],
        a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), px.ERR_INVALID_ARG),
    (dict(v=None), px.ERR_INVALID_ARG),
    (dict(rho=None), px.ERR_INVALID_ARG),
    (dict(out=None), px.ERR_INVALID_ARG),
    (dict(D=32), px.ERR_UNSUPPORTED),
    (dict(N=-1), px.ERR_INVALID_ARG),
    (dict(idt=3), px.ERR_INVALID_ARG),
    (dict(scale=float("nan")), px.ERR_INVALID_ARG),
    (dict(k=FAKE + 4), px.ERR_UNSUPPORTED),
    (dict(rs=(1, 16 * 128, 128)), px.ERR_UNSUPPORTED),
    (dict(os=(-1, 16 * 128, 128)), px.ERR_INVALID_ARG),
    # bf16 inputs need the packed-V workspace, B H ceil(N/64) 64 D 2 bytes
    (dict(ws=None, wsb=0), px.ERR_WORKSPACE),
    (dict(wsb=8 * 16 * 4096 * 128 * 2 - 1), px.ERR_WORKSPACE),
    (dict(ws=FAKE + 8), px.ERR_UNSUPPORTED),
])
def test_fwd_validation(lib, kw, status):
    assert _fwd(lib, **kw) == status


def test_fwd_workspace_size():
    # one fp16 64 x D tile per (b, h, 64-key block); none for fp32 inputs
    assert px.fwd_workspace_size(8, 4096, 16, 128) == 8 * 16 * 64 * 64 * 128 * 2
    assert px.fwd_workspace_size(2, 65, 3, 64) == 2 * 3 * 2 * 64 * 64 * 2
    assert px.fwd_workspace_size(2, 64, 3, 64) == 2 * 3 * 1 * 64 * 64 * 2
    assert px.fwd_workspace_size(1, 0, 1, 128) == 0
    import torch
    assert px.fwd_workspace_size(8, 4096, 16, 128, torch.float32) == 0
    with pytest.raises(px.ParallaxError):
        px.fwd_workspace_size(1, 64, 1, 96)



def test_fwd_empty_problem_is_ok(lib):
    assert _fwd(lib, N=0, q=None, k=None, v=None, rho=None, out=None) == px.OK


def test_python_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 2, 64)
    k = torch.zeros(1, 2, 8, 64)
    with pytest.raises(px.ParallaxError):
        px.decode(q, k, k, q)
    with pytest.raises(px.ParallaxError):
        px.fwd(k, k, k, k)


def test_python_binding_rejects_mixed_devices():
    """Tensors of one call must share a GPU, and an explicit stream must be
    on that GPU (host-side checks, before any device work)."""
    import torch

    class Dev:   # stands in for a device tensor or stream
        def __init__(self, index):
            self.is_cuda = True
            self.device = torch.device("cuda", index)

    px._need_gpu(Dev(0), None, Dev(0))
    with pytest.raises(px.ParallaxError, match="one GPU"):
        px._need_gpu(Dev(0), Dev(1))
    with pytest.raises(px.ParallaxError, match="another GPU"):
        px._stream(torch.device("cuda", 0), Dev(1))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(px.ParallaxError):
        px.library(str(tmp_path / "libparallax.so"))


def _gqa(lib, **kw):
    a = dict(q=FAKE, qs=(16 * 128, 128), rho=FAKE, rs=(16 * 128, 128), k=FAKE, v=FAKE,
             kvs=(4 * 4096 * 128, 4096 * 128, 128), bt=None, bt_sb=0, page=0, npages=0,
             sl=None, out=FAKE, os=(16 * 128, 128), B=2, Hq=16, Hkv=4, D=128, L=4096,
             scale=0.088, idt=px.BF16, odt=px.F32, ns=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.parallax_decode_gqa(
        a["q"], *a["qs"], a["rho"], *a["rs"], a["k"], a["v"], *a["kvs"], a["bt"],
        a["bt_sb"], a["page"], a["npages"], a["sl"], a["out"], *a["os"], a["B"], a["Hq"],
        a["Hkv"], a["D"], a["L"], a["scale"], a["idt"], a["odt"], a["ns"], a["ws"], a["wsb"],
        a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=12, Hkv=8), px.ERR_INVALID_ARG),      # not a multiple
    (dict(Hq=12, Hkv=4), px.ERR_UNSUPPORTED),      # group of 3
    (dict(Hkv=0), px.ERR_INVALID_ARG),
    (dict(idt=px.F32), px.ERR_UNSUPPORTED),
    (dict(D=96), px.ERR_UNSUPPORTED),
    (dict(bt=FAKE, page=12, npages=10, sl=FAKE), px.ERR_UNSUPPORTED),
    (dict(bt=FAKE, page=16, npages=10), px.ERR_INVALID_ARG),      # no seqlens
    (dict(bt=FAKE, page=16, npages=0, sl=FAKE), px.ERR_INVALID_ARG),
    (dict(bt=FAKE + 2, page=16, npages=10, sl=FAKE), px.ERR_UNSUPPORTED),
    (dict(ns=0), px.ERR_WORKSPACE),                 # 8 streams of 4096 keys split
    (dict(q=FAKE + 2), px.ERR_UNSUPPORTED),
])
def test_decode_gqa_validation(lib, kw, status):
    assert _gqa(lib, **kw) == status
    assert lib.parallax_last_error() != b""


def test_decode_gqa_workspace_size():
    # records per (b, query head, split); splits planned over B * Hkv streams
    s = px.decode_gqa_splits(2, 16, 4, 128, 4096)
    assert s == 32       # 8 streams: 32 splits wanted, at most 4096 / 128
    assert px.decode_gqa_splits(1, 32, 8, 128, 1024) == 8
    assert px.decode_gqa_splits(1, 32, 8, 128, 32768) == 32
    assert px.decode_gqa_splits(256, 32, 8, 128, 8192) == 1
    assert px.decode_gqa_splits(2, 16, 4, 128, 4096, 3) == 3
    rec = (4 + 2 * 128) * 4
    assert px.decode_gqa_workspace_size(2, 16, 4, 128, 4096) == 2 * 16 * s * rec
    assert px.decode_gqa_workspace_size(256, 32, 8, 128, 8192) == 0
    # workgroups of all 8 kv heads of a sequence: paged once sequences x
    # cache length reach 2^17 (splits then aim at 256 such workgroups),
    # contiguous only when 256 sequences need no split
    assert px.decode_gqa_splits(64, 32, 8, 128, 8192, paged=True) == 4
    assert px.decode_gqa_splits(64, 32, 8, 128, 8192) == 1          # 512 streams
    assert px.decode_gqa_splits(8, 32, 8, 128, 32768, paged=True) == 32
    assert px.decode_gqa_splits(8, 32, 8, 128, 32768) == 4          # 64 streams
    assert px.decode_gqa_splits(1, 32, 8, 128, 8192, paged=True) == 32   # below 2^17
    assert px.decode_gqa_splits(256, 32, 8, 128, 8192, paged=True) == 1
    # paged groups of fewer than 4 kv heads keep one kv head per workgroup:
    # the plan is the contiguous one's
    for B, Hq, Hkv, L in ((64, 8, 1, 8192), (128, 16, 2, 8192), (64, 48, 6, 8192)):
        assert (px.decode_gqa_splits(B, Hq, Hkv, 128, L, paged=True)
                == px.decode_gqa_splits(B, Hq, Hkv, 128, L))
    assert px.decode_gqa_splits(128, 32, 4, 128, 8192, paged=True) == 4
    assert px.decode_gqa_workspace_size(64, 32, 8, 128, 8192, paged=True) == 64 * 32 * 4 * rec
    assert px.decode_gqa_workspace_size(64, 32, 8, 128, 8192) == 0


@pytest.mark.parametrize("args,status", [
    ((FAKE, 1024, None), px.ERR_INVALID_ARG),      # no sink
    ((None, 1024, FAKE), px.ERR_INVALID_ARG),      # no source
    ((FAKE, -16, FAKE), px.ERR_INVALID_ARG),
    ((FAKE, 1000, FAKE), px.ERR_UNSUPPORTED),      # not a multiple of 16
    ((FAKE + 8, 1024, FAKE), px.ERR_UNSUPPORTED),  # misaligned source
    ((FAKE, 1024, FAKE + 2), px.ERR_UNSUPPORTED),  # misaligned sink
])
def test_stream_read_validation(lib, args, status):
    assert lib.parallax_stream_read(*args, None) == status
    assert lib.parallax_last_error() != b""


def _varlen(lib, **kw):
    s = (16 * 128, 128)
    a = dict(q=FAKE, k=FAKE, v=FAKE, rho=FAKE, out=FAKE, qs=s, ks=s, vs=s, rs=s, os=s,
             cu=FAKE, B=8, maxlen=4096, H=16, D=128, scale=0.088, causal=1,
             idt=px.BF16, odt=px.F32, ws=FAKE, wsb=8 * 16 * 4096 * 128 * 2, stream=None)
    a.update(kw)
    return lib.parallax_fwd_varlen(
        a["q"], *a["qs"], a["k"], *a["ks"], a["v"], *a["vs"], a["rho"], *a["rs"],
        a["out"], *a["os"], a["cu"], a["B"], a["maxlen"], a["H"], a["D"], a["scale"],
        a["causal"], a["idt"], a["odt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), px.ERR_INVALID_ARG),
    (dict(cu=FAKE + 2), px.ERR_UNSUPPORTED),
    (dict(idt=px.F32), px.ERR_UNSUPPORTED),
    (dict(q=None), px.ERR_INVALID_ARG),
    (dict(rho=FAKE + 4), px.ERR_UNSUPPORTED),
    (dict(D=96), px.ERR_UNSUPPORTED),
    (dict(maxlen=-1), px.ERR_INVALID_ARG),
    (dict(B=-2), px.ERR_INVALID_ARG),
    (dict(scale=float("inf")), px.ERR_INVALID_ARG),
    (dict(ws=None, wsb=0), px.ERR_WORKSPACE),
    (dict(wsb=100), px.ERR_WORKSPACE),
    (dict(ws=FAKE + 8), px.ERR_UNSUPPORTED),
    (dict(ks=(1 << 24, 128), maxlen=1 << 12), px.ERR_UNSUPPORTED),   # > 2 GiB per sequence
])
def test_fwd_varlen_validation(lib, kw, status):
    assert _varlen(lib, **kw) == status
    assert lib.parallax_last_error() != b""


def test_fwd_varlen_empty_is_ok(lib):
    assert _varlen(lib, B=0, q=None, ws=None, wsb=0) == px.OK
    assert _varlen(lib, maxlen=0, ws=None, wsb=0) == px.OK


def _proj(lib, **kw):
    a = dict(x=FAKE, xs=2048, w=FAKE, ws=2048, y=FAKE, ys=8192, M=32768, N=8192, K=2048,
             dt=px.BF16, stream=None)
    a.update(kw)
    return lib.parallax_project(a["x"], a["xs"], a["w"], a["ws"], a["y"], a["ys"], a["M"],
                                a["N"], a["K"], a["dt"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), px.ERR_INVALID_ARG),
    (dict(y=None), px.ERR_INVALID_ARG),
    (dict(M=-1), px.ERR_INVALID_ARG),
    (dict(dt=px.F32), px.ERR_UNSUPPORTED),
    (dict(N=8000, ys=8000), px.ERR_UNSUPPORTED),       # N not a multiple of 256
    (dict(K=2000, xs=2000, ws=2000), px.ERR_UNSUPPORTED),
    (dict(K=0), px.ERR_UNSUPPORTED),
    (dict(xs=1024), px.ERR_INVALID_ARG),                # stride shorter than a row
    (dict(ys=4096), px.ERR_INVALID_ARG),
    (dict(w=FAKE + 8), px.ERR_UNSUPPORTED),
    (dict(xs=2052), px.ERR_UNSUPPORTED),                # 16-byte row stride
    (dict(xs=1 << 23), px.ERR_UNSUPPORTED),             # 32-bit block offsets
])
def test_project_validation(lib, kw, status):
    assert _proj(lib, **kw) == status
    assert lib.parallax_last_error() != b""


def test_project_empty_is_ok(lib):
    assert _proj(lib, M=0, x=None) == px.OK


def _fwd_train(lib, **kw):
    s = (4096 * 16 * 128, 16 * 128, 128)
    a = dict(q=FAKE, k=FAKE, v=FAKE, rho=FAKE, out=FAKE, vbar=FAKE, lr=FAKE, s=s, B=8,
             N=4096, H=16, D=128, scale=0.088, causal=1, idt=px.BF16, odt=px.F32, ws=FAKE,
             wsb=8 * 16 * 4096 * 128 * 2, stream=None)
    a.update(kw)
    return lib.parallax_fwd_train(
        a["q"], *a["s"], a["k"], *a["s"], a["v"], *a["s"], a["rho"], *a["s"], a["out"],
        *a["s"], a["vbar"], a["lr"], a["B"], a["N"], a["H"], a["D"], a["scale"],
        a["causal"], a["idt"], a["odt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(vbar=None), px.ERR_INVALID_ARG),
    (dict(lr=None), px.ERR_INVALID_ARG),
    (dict(vbar=FAKE + 4), px.ERR_UNSUPPORTED),
    (dict(lr=FAKE + 4), px.ERR_UNSUPPORTED),
    (dict(idt=px.F32), px.ERR_UNSUPPORTED),
    (dict(q=None), px.ERR_INVALID_ARG),
    (dict(ws=None, wsb=0), px.ERR_WORKSPACE),
])
def test_fwd_train_validation(lib, kw, status):
    assert _fwd_train(lib, **kw) == status
    assert lib.parallax_last_error() != b""


def _bwd_saved(lib, **kw):
    s = (4096 * 16 * 128, 16 * 128, 128)
    a = dict(out=FAKE, odt=px.F32, vbar=FAKE, lr=FAKE, B=8, N=4096, H=16, D=128,
             idt=px.BF16, ws=FAKE, wsb=1 << 34, stream=None)
    a.update(kw)
    ptrs = [FAKE, *s] * 5                       # q, k, v, rho, dout
    return lib.parallax_bwd_saved(
        *ptrs, a["out"], *s, a["odt"], a["vbar"], a["lr"], *([FAKE, *s] * 4), a["B"],
        a["N"], a["H"], a["D"], 0.088, 1, a["idt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(out=None), px.ERR_INVALID_ARG),
    (dict(vbar=None), px.ERR_INVALID_ARG),
    (dict(lr=None), px.ERR_INVALID_ARG),
    (dict(lr=FAKE + 4), px.ERR_UNSUPPORTED),
    (dict(vbar=FAKE + 4), px.ERR_UNSUPPORTED),        # read with 16-byte loads
    (dict(out=FAKE + 8), px.ERR_UNSUPPORTED),
    (dict(odt=9), px.ERR_INVALID_ARG),
    (dict(idt=px.F32), px.ERR_UNSUPPORTED),
    (dict(ws=None, wsb=0), px.ERR_WORKSPACE),
])
def test_bwd_saved_validation(lib, kw, status):
    assert _bwd_saved(lib, **kw) == status
    assert lib.parallax_last_error() != b""


@pytest.mark.parametrize("call,kw", [
    ("fwd", dict(B=70000)),
    ("fwd", dict(H=70000)),
    ("decode", dict(B=70000)),
    ("varlen", dict(B=70000)),
    ("bwd_saved", dict(B=70000)),
    # 12 kv heads: three workgroups of 4 kv heads per sequence, 3 * 2^30
    ("gqa", dict(B=1 << 30, Hq=48, Hkv=12, kvs=(12 * 4096 * 128, 4096 * 128, 128))),
])
def test_oversized_launch_grid_is_unsupported(lib, call, kw):
    fn = {"fwd": _fwd, "decode": _decode, "varlen": _varlen, "bwd_saved": _bwd_saved,
          "gqa": _gqa}[call]
    assert fn(lib, **kw) == px.ERR_UNSUPPORTED
    assert b"grid" in lib.parallax_last_error()


def test_decode_noalloc_host_validation(lib):
    """parallax_decode_noalloc validates like parallax_decode and refuses,
    before any HIP call, split records beyond its 4 MiB device scratch."""
    args = lambda q, B, H, L, ns: (q, 16 * 128 * 16, 128, FAKE, 16 * 128 * 16, 128,
                                   FAKE, FAKE, 16 * L * 128, L * 128, 128, None,
                                   FAKE, 16 * 128, 128, B, H, 128, L,
                                   ctypes.c_float(0.1), px.BF16, px.F32, ns, None)
    assert lib.parallax_decode_noalloc(*args(None, 16, 16, 4096, 0)) == px.ERR_INVALID_ARG
    st = lib.parallax_decode_noalloc(*args(FAKE, 16, 16, 4096, 64))
    assert st == px.ERR_WORKSPACE
    assert b"4194304" in lib.parallax_last_error()
    # the library's own plan for a small batch fits (256 records of 1040 B)
    assert px.decode_workspace_size(1, 16, 128, 32768) <= 4 << 20
