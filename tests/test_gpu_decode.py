"""GPU parity of parallax_decode against the fp64 oracle (through the C ABI).

Inputs come from ``synth`` (seeded, drawn on the GPU); the oracle receives
host copies of exactly the tensors the kernel consumed. Tolerances: max abs
error 1e-4 for fp32 inputs, 2e-2 for bf16 inputs (fp32 accumulation, fp32
output), as stated for this path.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import transformer_attention_parallax_amd as px
from gpu_helpers import announce, max_abs_err, poison_cache_tail, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _oracle_decode(inp, scale=None, bh=None):
    """Oracle on all (b, h) or on the listed (b, h) pairs; returns float64."""
    q, rho, k, v, sl = (inp[n] for n in ("q", "rho", "k", "v", "seqlens"))
    if bh is None:
        return oracle.decode(q.cpu(), rho.cpu(), k.cpu(), v.cpu(),
                             seqlens=sl.cpu(), scale=scale)
    outs = []
    for b, h in bh:
        n = int(sl[b].item())
        outs.append(oracle.decode(
            q[b:b + 1, h:h + 1].cpu(), rho[b:b + 1, h:h + 1].cpu(),
            k[b:b + 1, h:h + 1, :max(n, 1)].cpu(),
            v[b:b + 1, h:h + 1, :max(n, 1)].cpu(),
            seqlens=np.array([n], np.int32), scale=scale)[0, 0])
    return np.stack(outs)


def test_decode_small_workload():
    shp = synth.WORKLOADS["decode_small"]
    announce("decode_small", shp)
    inp = synth.decode_inputs(shp, device=DEV)
    out = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"], inp["seqlens"])
    torch.cuda.synchronize()
    ref = _oracle_decode(inp)
    err = max_abs_err(out, ref)
    print(f"decode_small max abs err {err:.3e}", flush=True)
    assert err <= tol_for(shp.dtype)


def test_decode_small_workload_rho_zero_is_softmax():
    shp = synth.WORKLOADS["decode_small"]
    announce("decode_small rho=0", shp)
    inp = synth.decode_inputs(shp, device=DEV, rho_zero=True)
    out = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"], inp["seqlens"])
    torch.cuda.synchronize()
    ref = _oracle_decode(inp)
    assert max_abs_err(out, ref) <= tol_for(shp.dtype)
    # plain softmax attention from torch on the same values, fp32 on the CPU
    q = inp["q"].float().cpu()[:, :, None, :]
    sdpa = torch.nn.functional.scaled_dot_product_attention(
        q, inp["k"].float().cpu(), inp["v"].float().cpu(),
        scale=1.0 / math.sqrt(shp.D))[:, :, 0, :]
    assert max_abs_err(out, sdpa.double().numpy()) <= tol_for(shp.dtype)


@pytest.mark.parametrize("splits", [1, 2, 7, 32, 64])
def test_decode_split_invariance(splits):
    shp = synth.WORKLOADS["decode_small"]
    announce("decode split invariance", splits)
    inp = synth.decode_inputs(shp, device=DEV)
    base = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"], inp["seqlens"],
                     num_splits=1)
    out = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"], inp["seqlens"],
                    num_splits=splits)
    torch.cuda.synchronize()
    assert px.decode_splits(shp.B, shp.H, shp.D, shp.L, splits) == splits
    assert torch.max(torch.abs(out - base)).item() <= 1e-5
    ref = _oracle_decode(inp, bh=[(0, 0), (0, 7), (0, 15)])
    assert max_abs_err(out[0, [0, 7, 15]], ref) <= tol_for(shp.dtype)


@pytest.mark.parametrize("D,L,splits", [(64, 6400, 100), (128, 12800, 200),
                                          (64, 65536, 1024)])
def test_decode_many_splits(D, L, splits):
    # more splits than the combine has threads (each thread merges several
    # splits' scalars), up to the largest split count a call may use
    shp = synth.DecodeShape(B=1, H=2, D=D, L=L, index=6)
    announce("decode many splits", D, L, splits)
    inp = synth.decode_inputs(shp, device=DEV)
    assert px.decode_splits(1, 2, D, L, splits) == splits
    base = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"], inp["seqlens"],
                     num_splits=1)
    out = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"], inp["seqlens"],
                    num_splits=splits)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(out - base)).item() <= 1e-5
    ref = _oracle_decode(inp, bh=[(0, 0), (0, 1)])
    assert max_abs_err(out[0], ref) <= tol_for(shp.dtype)


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_decode_ragged_poisoned(splits):
    shp = synth.DecodeShape(B=6, H=4, D=128, L=777, index=40)
    announce("decode ragged poisoned", splits)
    inp = synth.decode_inputs(shp, device=DEV)
    inp["seqlens"] = torch.tensor([777, 0, 1, 300, 64, 513], dtype=torch.int32,
                                  device=DEV)
    poison_cache_tail(inp["k"], inp["seqlens"])
    poison_cache_tail(inp["v"], inp["seqlens"])
    out = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"], inp["seqlens"],
                    num_splits=splits)
    torch.cuda.synchronize()
    ref = _oracle_decode(inp)
    assert max_abs_err(out, ref) <= tol_for(shp.dtype)
    assert torch.count_nonzero(out[1]).item() == 0  # empty context -> zeros


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_dtypes_and_head_dims(dtype, D):
    shp = synth.DecodeShape(B=3, H=2, D=D, L=1000, dtype=dtype, index=41)
    announce("decode dtype/D", dtype, D)
    inp = synth.decode_inputs(shp, device=DEV, ragged=True)
    for splits in (1, 0, 5):
        out = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"],
                        inp["seqlens"], num_splits=splits)
        torch.cuda.synchronize()
        ref = _oracle_decode(inp)
        err = max_abs_err(out, ref)
        assert err <= tol_for(dtype), (splits, err)
        # bf16 output is the RNE rounding of the same fp32 result
        ob = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"],
                       inp["seqlens"], num_splits=splits,
                       out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(ob, out.to(torch.bfloat16))


def test_decode_strided_cache_and_scale():
    """Cache stored [B, L, H, D] and viewed as [B, H, L, D]; q, rho slices."""
    B, H, L, D = 2, 3, 517, 128
    announce("decode strided cache")
    g = synth.gen(4242, DEV)
    kc = torch.randn(B, L, H, D, device=DEV, generator=g).to(torch.bfloat16)
    vc = torch.randn(B, L, H, D, device=DEV, generator=g).to(torch.bfloat16)
    qr = torch.randn(B, H, 2 * D, device=DEV, generator=g).to(torch.bfloat16)
    q, rho = qr[:, :, :D], (0.3 * qr[:, :, D:].float()).to(torch.bfloat16)
    k, v = kc.permute(0, 2, 1, 3), vc.permute(0, 2, 1, 3)
    assert k.stride(2) == H * D
    sl = torch.tensor([517, 200], dtype=torch.int32, device=DEV)
    out = px.decode(q, k, v, rho, sl, scale=0.05)
    torch.cuda.synchronize()
    ref = oracle.decode(q.cpu(), rho.cpu(), k.cpu(), v.cpu(), seqlens=sl.cpu(),
                        scale=0.05)
    assert max_abs_err(out, ref) <= 2e-2


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 127, 129, 4097])
def test_decode_edge_lengths(L):
    shp = synth.DecodeShape(B=2, H=2, D=128, L=L, index=42)
    announce("decode edge length", L)
    inp = synth.decode_inputs(shp, device=DEV)
    for splits in (0, 1, 2):
        out = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"],
                        inp["seqlens"], num_splits=splits)
        torch.cuda.synchronize()
        assert max_abs_err(out, _oracle_decode(inp)) <= 2e-2
    if L == 1:  # a single key returns its value
        o = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"])
        torch.cuda.synchronize()
        assert torch.equal(o, inp["v"][:, :, 0].float())


def test_decode_large_workload_sampled():
    """Full-size 256 x 16 x 8192 bf16 cache, sampled (b, h) vs the oracle."""
    shp = synth.WORKLOADS["decode_large"]
    announce("decode_large", shp)
    inp = synth.decode_inputs(shp, device=DEV)
    out = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"], inp["seqlens"])
    torch.cuda.synchronize()
    bh = [(0, 0), (0, 15), (17, 3), (100, 8), (128, 0), (200, 11), (254, 7),
          (255, 15)]
    rng = np.random.default_rng(3003)   # plus 120 seeded random streams
    bh += [(int(b), int(h)) for b, h in zip(rng.integers(0, shp.B, 120),
                                             rng.integers(0, shp.H, 120))]
    ref = _oracle_decode(inp, bh=bh)
    got = torch.stack([out[b, h] for b, h in bh])
    err = max_abs_err(got, ref)
    print(f"decode_large sampled max abs err {err:.3e}", flush=True)
    assert err <= tol_for(shp.dtype)
    assert torch.isfinite(out).all().item()
    del inp
    torch.cuda.empty_cache()


SWEEP = synth.sweep_points()
FULL_CHECK_TOKENS = 1 << 21  # up to this many cache rows per head: 3 batch rows x all heads


def _sweep_streams(B, L):
    """(b, h) streams compared with the oracle at one sweep point: the first,
    middle and last sequence in every head (all 16 heads at short contexts),
    plus, on the large points, seeded random streams across the batch."""
    bs = sorted({0, B // 2, B - 1})
    hs = [0, 5, 15] if L >= 8192 else list(range(16))
    bh = [(b, h) for b in bs for h in hs]
    if B * L > FULL_CHECK_TOKENS:
        g = np.random.default_rng(1000 * 4 + B + L)
        extra = zip(g.integers(0, B, 12), g.integers(0, 16, 12))
        bh += [(int(b), int(h)) for b, h in extra if (int(b), int(h)) not in bh]
    return bh


@pytest.mark.parametrize("ragged", [False, True])
@pytest.mark.parametrize("B,L", SWEEP)
def test_decode_sweep_point(B, L, ragged):
    """Every point of the batch x context decode grid (up to the 2048 x 8192
    cache of 137 GB), uniform and ragged lengths; ragged caches hold NaN past
    each length. The launch is the one bench.py's sweep times (library's
    split plan); sampled (b, h) streams go to the oracle on host slices."""
    shp = synth.DecodeShape(B=B, H=16, D=128, L=L, index=4)
    announce("decode sweep", B, L, "ragged" if ragged else "uniform")
    inp = synth.decode_inputs(shp, device=DEV, ragged=ragged)
    if ragged:
        poison_cache_tail(inp["k"], inp["seqlens"])
        poison_cache_tail(inp["v"], inp["seqlens"])
    out = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"], inp["seqlens"])
    torch.cuda.synchronize()
    bh = _sweep_streams(B, L)
    ref = _oracle_decode(inp, bh=bh)
    got = torch.stack([out[b, h] for b, h in bh])
    err = max_abs_err(got, ref)
    print(f"decode sweep {B}x{L} {'ragged' if ragged else 'uniform'}: "
          f"{len(bh)} streams, max abs err {err:.3e}", flush=True)
    assert err <= 2e-2
    assert torch.isfinite(out).all().item()
    del inp, out
    torch.cuda.empty_cache()


def test_decode_negative_scale_and_growing_scores():
    B, H, L, D = 2, 3, 3000, 128
    announce("decode negative scale / growing scores")
    g = synth.gen(9002, DEV)
    grow = torch.linspace(0.2, 3.0, L, device=DEV).view(1, 1, L, 1)
    k = (torch.randn(B, H, L, D, device=DEV, generator=g) * grow).to(torch.bfloat16)
    v = torch.randn(B, H, L, D, device=DEV, generator=g).to(torch.bfloat16)
    q = (2.0 * torch.randn(B, H, D, device=DEV, generator=g)).to(torch.bfloat16)
    rho = (0.1 * torch.randn(B, H, D, device=DEV, generator=g)).to(torch.bfloat16)
    for scale in (0.2, -0.2):
        for splits in (0, 1, 4):
            out = px.decode(q, k, v, rho, scale=scale, num_splits=splits)
            torch.cuda.synchronize()
            ref = oracle.decode(q.cpu(), rho.cpu(), k.cpu(), v.cpu(), scale=scale)
            assert max_abs_err(out, ref) <= 2e-2, (scale, splits)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("splits", [1, 5])
def test_decode_softmax_only(dtype, splits):
    """rho = NULL: plain softmax attention, bit-equal to rho = 0 (the probe
    sums are skipped, and with rho = 0 they are exactly zero) and within the
    bar of the oracle's softmax attention."""
    shp = synth.DecodeShape(B=3, H=4, D=128, L=777, dtype=dtype, index=2)
    announce("decode softmax only", dtype, splits)
    inp = synth.decode_inputs(shp, device=DEV, ragged=True, seed_base=41)
    inp["rho"] = torch.zeros_like(inp["q"])
    a = px.decode(inp["q"], inp["k"], inp["v"], None, inp["seqlens"], num_splits=splits)
    b = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"], inp["seqlens"],
                  num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = _oracle_decode(inp)          # the oracle at rho = 0 is softmax attention
    assert max_abs_err(a, ref) <= tol_for(dtype)


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 16, (64 << 20) + 48])
def test_stream_read_checksum(nbytes):
    """parallax_stream_read folds every 32-bit word with XOR: equal to the
    host XOR of the same bytes, so every byte was read exactly once."""
    announce("stream read", nbytes)
    g = synth.gen(990 + nbytes % 97, DEV)
    n = nbytes // 4
    src = torch.randint(-(1 << 31), (1 << 31) - 1, (max(n, 4),), dtype=torch.int32,
                        device=DEV, generator=g)[:n]
    sink = torch.full((1,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    px.stream_read(src, sink)
    torch.cuda.synchronize()
    host = src.cpu().numpy().view(np.uint32)
    want = np.uint32(0x5A5A5A5A)
    if host.size:
        want ^= np.bitwise_xor.reduce(host)
    assert np.uint32(sink.cpu().numpy().view(np.uint32)[0]) == want


@pytest.mark.parametrize("splits", [2, 16, 300])
def test_decode_split_workspace_garbage_and_reuse(splits):
    """The split records' workspace needs no initialisation: a workspace
    filled with NaN bytes and reused by repeated calls gives bit-identical
    outputs within the bar of the oracle; a bf16 output is the RNE rounding
    of the fp32 one."""
    shp = synth.DecodeShape(B=3, H=5, D=128, L=20000, index=43)
    announce("decode split workspace", splits)
    inp = synth.decode_inputs(shp, device=DEV, ragged=True)
    need = px.decode_workspace_size(shp.B, shp.H, shp.D, shp.L, splits)
    ws = torch.full((need // 4 + 16,), float("nan"), device=DEV).view(torch.uint8)
    outs = []
    for _ in range(3):
        outs.append(px.decode(inp["q"], inp["k"], inp["v"], inp["rho"], inp["seqlens"],
                              num_splits=splits, workspace=ws))
        torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
    ref = _oracle_decode(inp, bh=[(0, 0), (1, 4), (2, 2)])
    got = torch.stack([outs[0][b, h] for b, h in [(0, 0), (1, 4), (2, 2)]])
    assert max_abs_err(got, ref) <= 2e-2
    ob = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"], inp["seqlens"],
                   num_splits=splits, workspace=ws, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(ob, outs[0].to(torch.bfloat16))
