"""GPU parity of parallax_project (the fused q, k, v, rho input projection)
against the fp64 oracle product, through the C ABI.

Bar: the output is the fp32-accumulated product rounded to bf16, so per
element |y - ref| <= 2^-8 |ref| (one bf16 rounding, relative 2^-9, with
margin) + 2^-16 sum_k |x_k w_k| (fp32 accumulation over K terms in another
order than the oracle's).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import transformer_attention_parallax_amd as px
from gpu_helpers import announce, max_abs_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check(y, x, w, rows=None):
    xh = x.double().cpu().numpy()
    wh = w.double().cpu().numpy()
    if rows is not None:
        xh = xh[rows]
        y = y[torch.as_tensor(rows, device=y.device)]
    ref = oracle.project(xh, wh)
    mag = np.abs(xh) @ np.abs(wh).T
    got = y.double().cpu().numpy()
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * mag
    excess = np.abs(got - ref) - bound
    assert np.isfinite(got).all()
    assert excess.max() <= 0.0, (float(np.abs(got - ref).max()), float(excess.max()))
    return float(np.abs(got - ref).max())


@pytest.mark.parametrize("M,N,K", [(1, 256, 64), (100, 512, 192), (256, 256, 128),
                                   (300, 768, 64), (1000, 512, 512), (513, 1024, 256)])
def test_project_shapes(M, N, K):
    announce("project", M, N, K)
    g = synth.gen(1200 + M + N + K, DEV)
    x = torch.randn(M, K, device=DEV, generator=g).to(torch.bfloat16)
    w = (0.05 * torch.randn(N, K, device=DEV, generator=g)).to(torch.bfloat16)
    y = px.project(x, w)
    torch.cuda.synchronize()
    _check(y, x, w)


def test_project_strided_views():
    """x a column slice of a wider tensor, y written into a slice of a wider
    buffer whose other columns stay untouched."""
    M, N, K = 333, 512, 128
    announce("project strided")
    g = synth.gen(1210, DEV)
    xb = torch.randn(M, K + 64, device=DEV, generator=g).to(torch.bfloat16)
    x = xb[:, 32:32 + K]
    w = (0.05 * torch.randn(N, K, device=DEV, generator=g)).to(torch.bfloat16)
    yb = torch.full((M, N + 256), float("nan"), device=DEV).to(torch.bfloat16)
    px.project(x, w, out=yb[:, 128:128 + N])
    torch.cuda.synchronize()
    _check(yb[:, 128:128 + N], x, w)
    assert torch.isnan(yb[:, :128].float()).all().item()
    assert torch.isnan(yb[:, 128 + N:].float()).all().item()


def test_project_zero_wr_gives_softmax_attention():
    """A converted layer (W_R = 0 stacked by fuse_qkvr_weight): the probe is
    exactly zero and the Parallax output is plain softmax attention (torch
    SDPA in fp32 on the CPU)."""
    B, N, Hq, Hkv, D, dm = 1, 200, 4, 4, 64, 256
    announce("project W_R = 0")
    g = synth.gen(1220, DEV)
    x = torch.randn(B * N, dm, device=DEV, generator=g).to(torch.bfloat16)
    wq, wk, wv = ((torch.randn(Hq * D, dm, device=DEV, generator=g) / math.sqrt(dm))
                  .to(torch.bfloat16) for _ in range(3))
    w = px.fuse_qkvr_weight(wq, wk, wv)
    y = px.project(x, w)
    q, k, v, rho = px.split_qkvr(y, Hq, Hkv, D)
    assert torch.equal(rho.float(), torch.zeros_like(rho.float()))
    out = px.fwd(*(t.view(B, N, -1, D) for t in (q, k, v, rho)), causal=True)
    torch.cuda.synchronize()
    tt = [t.view(B, N, -1, D).float().cpu().transpose(1, 2) for t in (q, k, v)]
    sdpa = torch.nn.functional.scaled_dot_product_attention(*tt, is_causal=True,
                                                            scale=1.0 / math.sqrt(D))
    assert max_abs_err(out, sdpa.transpose(1, 2).double().numpy()) <= 2e-2


def test_project_then_attention_matches_oracle():
    """x -> project -> strided q, k, v, rho views -> parallax_fwd, against the
    oracle on the projection outputs the kernel read."""
    B, N, H, D, dm = 2, 130, 2, 128, 512
    announce("project + fwd")
    g = synth.gen(1230, DEV)
    x = torch.randn(B * N, dm, device=DEV, generator=g).to(torch.bfloat16)
    wq, wk, wv = ((torch.randn(H * D, dm, device=DEV, generator=g) / math.sqrt(dm))
                  .to(torch.bfloat16) for _ in range(3))
    wr = (0.02 * torch.randn(H * D, dm, device=DEV, generator=g)).to(torch.bfloat16)
    y = px.project(x, px.fuse_qkvr_weight(wq, wk, wv, wr))
    q, k, v, rho = (t.view(B, N, H, D) for t in px.split_qkvr(y, H, H, D))
    out = px.fwd(q, k, v, rho, causal=True)
    torch.cuda.synchronize()
    ref = oracle.fwd(*(t.cpu() for t in (q, k, v, rho)), causal=True)
    assert max_abs_err(out, ref) <= 2e-2


def test_project_full_size_sampled():
    """The 1.7B-shape projection: 8 x 4096 tokens of width 2048 onto
    q, k, v, rho of 16 heads x 128 (N = 8192); sampled rows."""
    shp = synth.WORKLOADS["project_qkvr"]
    announce("project full size", shp)
    inp = synth.project_inputs(shp, device=DEV)
    y = px.project(inp["x"], inp["w"])
    torch.cuda.synchronize()
    rows = np.random.default_rng(3).choice(shp.M, size=48, replace=False)
    rows = np.concatenate([rows, [0, shp.M - 1]])
    _check(y, inp["x"], inp["w"], rows=rows)
    del inp, y
    torch.cuda.empty_cache()
