"""GPU parity of parallax_fwd_varlen (packed variable-length prefill, bf16)
against the fp64 oracle, through the C ABI.

Each sequence of the packed batch is handed to the oracle as its own
[1, L, H, D] problem (host copies of exactly the tensors the GPU read); no
new oracle arithmetic is involved. Tolerance 2e-2 as for the bf16 prefill.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import transformer_attention_parallax_amd as px
from gpu_helpers import announce, max_abs_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2


def _packed(lens, H, D, seed, lead=0, tail=0, rho_std=0.1):
    """Packed [T, H, D] bf16 tensors with sequences at cu_seqlens (starting
    at row `lead`, `tail` spare rows after the last)."""
    g = synth.gen(seed, DEV)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64) + lead
    T = int(cu[-1]) + tail
    mk = lambda s=1.0: (s * torch.randn(T, H, D, device=DEV, generator=g)).to(torch.bfloat16)
    q, k, v, rho = mk(), mk(), mk(), mk(rho_std)
    return q, k, v, rho, torch.tensor(cu, dtype=torch.int32, device=DEV)


def _check(out, q, k, v, rho, cu, lens, causal=True, cut=None):
    for b, L in enumerate(lens):
        L = min(L, cut) if cut is not None else L
        if L == 0:
            continue
        a = int(cu[b])
        sl = slice(a, a + L)
        ref = oracle.fwd(*(t[sl].unsqueeze(0).cpu() for t in (q, k, v, rho)), causal=causal)
        err = max_abs_err(out[sl].unsqueeze(0), ref)
        assert err <= TOL, (b, L, err)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D", [64, 128])
def test_varlen_ragged(D, causal):
    lens = [17, 0, 1, 130, 64, 65, 300, 128, 129]
    H = 2
    announce("fwd varlen", D, causal)
    q, k, v, rho, cu = _packed(lens, H, D, seed=1100 + D, lead=3, tail=5)
    out = torch.full(q.shape, float("nan"), device=DEV)
    px.fwd_varlen(q, k, v, rho, cu, max(lens), causal=causal, out=out)
    torch.cuda.synchronize()
    _check(out, q, k, v, rho, cu.cpu(), lens, causal)
    # rows outside every sequence are not written
    assert torch.isnan(out[:3]).all().item() and torch.isnan(out[-5:]).all().item()


def test_varlen_equal_lengths_match_fwd():
    """Equal lengths: the packed call is parallax_fwd on [B, N, H, D] with
    other base offsets, bit for bit."""
    B, N, H, D = 3, 200, 2, 128
    announce("fwd varlen == fwd")
    q, k, v, rho, cu = _packed([N] * B, H, D, seed=1110)
    a = px.fwd_varlen(q, k, v, rho, cu, N)
    b = px.fwd(*(t.view(B, N, H, D) for t in (q, k, v, rho)), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(B, N, H, D), b)


def test_varlen_lengths_cut_at_max_seqlen():
    lens = [100, 40]
    H, D = 2, 64
    announce("fwd varlen cut")
    q, k, v, rho, cu = _packed(lens, H, D, seed=1120)
    out = torch.full(q.shape, float("nan"), device=DEV)
    px.fwd_varlen(q, k, v, rho, cu, 64, out=out)
    torch.cuda.synchronize()
    _check(out, q, k, v, rho, cu.cpu(), lens, cut=64)
    assert torch.isnan(out[64:100]).all().item()          # past the cut: untouched


def test_varlen_bf16_out_and_strided_views():
    """q, k, v from one fused [T, 3, H, D] tensor; bf16 output equals the
    RNE rounding of the fp32 output."""
    lens = [77, 190, 5]
    H, D = 3, 128
    announce("fwd varlen strided")
    g = synth.gen(1130, DEV)
    T = sum(lens)
    qkv = torch.randn(T, 3, H, D, device=DEV, generator=g).to(torch.bfloat16)
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    rho = (0.1 * torch.randn(T, H, D, device=DEV, generator=g)).to(torch.bfloat16)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    o32 = px.fwd_varlen(q, k, v, rho, cu, max(lens))
    o16 = px.fwd_varlen(q, k, v, rho, cu, max(lens), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))
    _check(o32, q, k, v, rho, cu.cpu(), lens)


def test_varlen_packed_workload_sampled():
    """The packed prefill workload (16 sequences, lengths 256..4096, 16
    heads, rho = x W_R): sampled (sequence, row, head) outputs."""
    shp = synth.WORKLOADS["prefill_varlen"]
    announce("fwd varlen workload", shp)
    inp = synth.varlen_prefill_inputs(shp, device=DEV)
    cu = inp["cu_seqlens"]
    out = px.fwd_varlen(inp["q"], inp["k"], inp["v"], inp["rho"], cu, shp.max_seqlen)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    cuh = cu.cpu().numpy()
    rng = np.random.default_rng(7)
    for b in rng.choice(len(cuh) - 1, size=4, replace=False):
        a, e = int(cuh[b]), int(cuh[b + 1])
        L = e - a
        rows = sorted({0, L - 1, *rng.integers(0, L, size=6).tolist()})
        sel = [(0, i, int(h)) for i in rows for h in rng.integers(0, shp.H, size=2)]
        ref = oracle.fwd_rows(*(t[a:e].unsqueeze(0).cpu() for t in
                                (inp["q"], inp["k"], inp["v"], inp["rho"])), sel)
        got = np.stack([out[a + i, h].double().cpu().numpy() for _, i, h in sel])
        assert np.abs(got - ref).max() <= TOL, (b, L)
