"""GPU parity of parallax_bwd (backward of the bf16 prefill) against the
fp64 oracle's gradients, through the C ABI.

Tolerance (per gradient tensor): max abs error <= 1e-2 * max |ref| + 1e-5.
The products q.k, rho.k and dout.v are exact bf16 products accumulated in
fp32; ds, dr and p (1 + rbar - r) enter the second contractions rounded to
bf16 (8-bit significand, relative rounding <= 2^-9 ~ 2.0e-3 per term), and
the probabilities are rebuilt from a log-sum-exp whose sum was taken over
fp16-rounded weights. Measured worst ratio over the cases below: 3.1e-3.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import transformer_attention_parallax_amd as px
from gpu_helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAMES = ("dq", "dk", "dv", "drho")


def _inputs(B, N, H, D, seed, rho_std=0.1):
    g = synth.gen(seed, DEV)
    mk = lambda s=1.0: (s * torch.randn(B, N, H, D, device=DEV, generator=g)).to(torch.bfloat16)
    return mk(), mk(), mk(), mk(rho_std), mk()


def _check(grads, ref, what=""):
    for name, a, r in zip(NAMES, grads, ref):
        a = a.double().cpu().numpy()
        assert np.isfinite(a).all(), f"{what} {name}: non-finite"
        err = float(np.abs(a - r).max())
        bound = 1e-2 * float(np.abs(r).max()) + 1e-5
        print(f"{what} {name}: err {err:.3e} bound {bound:.3e}", flush=True)
        assert err <= bound, (what, name, err, bound)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,N,H,D", [(1, 1, 1, 128), (1, 17, 2, 64), (1, 64, 1, 128),
                                     (2, 65, 2, 128), (1, 130, 2, 64), (2, 200, 3, 128)])
def test_bwd_shapes(B, N, H, D, causal):
    announce("bwd shape", B, N, H, D, causal)
    q, k, v, rho, dout = _inputs(B, N, H, D, seed=700 + N + D)
    grads = px.bwd(q, k, v, rho, dout, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.bwd(q.cpu(), k.cpu(), v.cpu(), rho.cpu(), dout.cpu(), causal=causal)
    _check(grads, ref, f"B{B} N{N} H{H} D{D} causal={causal}")


def test_bwd_strided_views_and_outputs():
    """q, k, v from one fused [B, N, 3, H, D] tensor; gradients written into
    strided views of one [B, N, 4, H, D] buffer."""
    B, N, H, D = 2, 150, 2, 128
    announce("bwd strided")
    g = synth.gen(811, DEV)
    qkv = torch.randn(B, N, 3, H, D, device=DEV, generator=g).to(torch.bfloat16)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    rho = (0.1 * torch.randn(B, N, H, D, device=DEV, generator=g)).to(torch.bfloat16)
    dout = torch.randn(B, N, H, D, device=DEV, generator=g).to(torch.bfloat16)
    buf = torch.full((B, N, 4, H, D), float("nan"), device=DEV)
    grads = [buf[:, :, i] for i in range(4)]
    px.bwd(q, k, v, rho, dout, causal=True, grads=grads)
    torch.cuda.synchronize()
    ref = oracle.bwd(q.cpu(), k.cpu(), v.cpu(), rho.cpu(), dout.cpu(), causal=True)
    _check(grads, ref, "strided")


@pytest.mark.parametrize("scale", [-0.15, 0.0, 0.3])
def test_bwd_scale(scale):
    B, N, H, D = 1, 96, 2, 64
    announce("bwd scale", scale)
    q, k, v, rho, dout = _inputs(B, N, H, D, seed=812)
    grads = px.bwd(q, k, v, rho, dout, causal=True, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.bwd(q.cpu(), k.cpu(), v.cpu(), rho.cpu(), dout.cpu(), scale=scale,
                     causal=True)
    _check(grads, ref, f"scale {scale}")


def test_bwd_large_probe():
    """rho = bf16(x W_R) with the 1.7B-shape recipe: |r| reaches tens."""
    shp = synth.PrefillShape(B=1, N=192, H=2, D=128, dtype=torch.bfloat16,
                             rho_from_x=True, index=813)
    announce("bwd large probe", shp)
    inp = synth.prefill_inputs(shp, device=DEV)
    g = synth.gen(814, DEV)
    dout = torch.randn(inp["q"].shape, device=DEV, generator=g).to(torch.bfloat16)
    grads = px.bwd(inp["q"], inp["k"], inp["v"], inp["rho"], dout, causal=True)
    torch.cuda.synchronize()
    ref = oracle.bwd(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["rho"].cpu(),
                     dout.cpu(), causal=True)
    _check(grads, ref, "large probe")


def test_bwd_rho_zero_matches_torch_autograd():
    """rho = 0 is softmax attention: dq, dk, dv against torch autograd of
    attention in fp32 on the CPU (drho against the oracle)."""
    B, N, H, D = 1, 80, 2, 128
    announce("bwd rho=0")
    q, k, v, _, dout = _inputs(B, N, H, D, seed=815)
    rho = torch.zeros_like(q)
    grads = px.bwd(q, k, v, rho, dout, causal=True)
    torch.cuda.synchronize()
    tt = [x.float().cpu().transpose(1, 2).contiguous().requires_grad_(True) for x in (q, k, v)]
    o = torch.nn.functional.scaled_dot_product_attention(*tt, is_causal=True,
                                                         scale=1.0 / math.sqrt(D))
    (o * dout.float().cpu().transpose(1, 2)).sum().backward()
    ref = [t.grad.transpose(1, 2).double().numpy() for t in tt]
    ref.append(oracle.bwd(q.cpu(), k.cpu(), v.cpu(), rho.cpu(), dout.cpu(), causal=True)[3])
    _check(grads, ref, "rho=0")


def test_bwd_deterministic_and_workspace_reuse():
    B, N, H, D = 2, 160, 2, 128
    announce("bwd determinism")
    q, k, v, rho, dout = _inputs(B, N, H, D, seed=816)
    ws = torch.full((px.bwd_workspace_size(B, N, H, D),), 255, dtype=torch.uint8, device=DEV)
    a = px.bwd(q, k, v, rho, dout, workspace=ws)
    b = px.bwd(q, k, v, rho, dout, workspace=ws)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_rejects_small_workspace_and_fp32():
    B, N, H, D = 1, 33, 1, 64
    q, k, v, rho, dout = _inputs(B, N, H, D, seed=817)
    small = torch.empty(px.bwd_workspace_size(B, N, H, D) - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(px.ParallaxError) as e:
        px.bwd(q, k, v, rho, dout, workspace=small)
    assert e.value.status == px.ERR_WORKSPACE
    f = [x.float() for x in (q, k, v, rho, dout)]
    with pytest.raises(px.ParallaxError) as e:
        px.bwd(*f)
    assert e.value.status == px.ERR_UNSUPPORTED


def test_bwd_full_size_invariants():
    """The 8 x 4096 x 16 x 128 causal workload: at any size the key
    gradients of each (b, h) sum to zero (a shift of every key changes no
    output), the value gradients sum to the output gradients (a shift of
    every value shifts every output), and rho_i . drho_i = g_i . (o_i - vbar_i)
    (the output is linear in rho), with o and vbar from the forward kernel."""
    shp = synth.WORKLOADS["prefill_bf16"]
    announce("bwd full size", shp)
    inp = synth.prefill_inputs(shp, device=DEV)
    g = synth.gen(818, DEV)
    dout = torch.randn(inp["q"].shape, device=DEV, generator=g).to(torch.bfloat16)
    dq, dk, dv, drho = px.bwd(inp["q"], inp["k"], inp["v"], inp["rho"], dout, causal=True)
    o = px.fwd(inp["q"], inp["k"], inp["v"], inp["rho"], causal=True)
    vbar = px.fwd(inp["q"], inp["k"], inp["v"], torch.zeros_like(inp["rho"]), causal=True)
    torch.cuda.synchronize()
    for t in (dq, dk, dv, drho):
        assert torch.isfinite(t).all().item()
    gs = dout.float()
    s_dk = dk.double().sum(dim=1)
    assert (s_dk.abs().max() / dk.double().abs().sum(dim=1).max()).item() < 1e-3
    s_dv = dv.double().sum(dim=1)
    ref_dv = gs.double().sum(dim=1)
    assert ((s_dv - ref_dv).abs().max() / ref_dv.abs().max()).item() < 1e-2
    lhs = (inp["rho"].float() * drho).sum(-1)
    rhs = (gs * (o - vbar)).sum(-1)
    err = (lhs - rhs).abs().max().item()
    print(f"full size: sum dk {s_dk.abs().max().item():.3e}, Euler err {err:.3e} "
          f"(max |rhs| {rhs.abs().max().item():.3e})", flush=True)
    assert err <= 2e-2 * rhs.abs().max().item() + 1e-3
    # element-wise: whole (b, h) heads (all 4096 queries and keys, every
    # causal pair) through the fp64 backward oracle on host slices
    for b, h in ((0, 0), (5, 11)):
        sl = lambda t: t[b:b + 1, :, h:h + 1].cpu()
        ref = oracle.bwd(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["rho"]), sl(dout),
                         causal=True)
        _check([t[b:b + 1, :, h:h + 1] for t in (dq, dk, dv, drho)], ref,
               f"full size head b={b} h={h}")
    del inp, dq, dk, dv, drho, o, vbar
    torch.cuda.empty_cache()


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,N,H,D,causal", [(1, 65, 2, 128, True), (2, 200, 3, 128, True),
                                            (1, 130, 2, 64, False)])
def test_bwd_saved_matches_oracle(B, N, H, D, causal, out_dtype):
    """Training forward + backward from its saved tensors: the output equals
    parallax_fwd bit for bit, vbar is the rho = 0 output of the oracle,
    {lse2, rbar} are the softmax log-normaliser and mean probe score, and the
    gradients meet the same bar as parallax_bwd."""
    announce("bwd saved", B, N, H, D, causal, out_dtype)
    q, k, v, rho, dout = _inputs(B, N, H, D, seed=830 + N + D)
    out, vbar, lr = px.fwd_train(q, k, v, rho, causal=causal, out_dtype=out_dtype)
    out_ref = px.fwd(q, k, v, rho, causal=causal, out_dtype=out_dtype)
    grads = px.bwd_saved(q, k, v, rho, dout, out, vbar, lr, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    vref = oracle.fwd(q.cpu(), k.cpu(), v.cpu(), torch.zeros_like(rho).cpu(), causal=causal)
    assert np.abs(vbar.double().cpu().numpy() - vref).max() <= 2e-2
    # lse2 and rbar from their definitions (fp64 numpy on the same values)
    qh, kh, rh = (t.double().cpu().numpy() for t in (q, k, rho))
    s = np.einsum("bihd,bjhd->bhij", qh, kh) / math.sqrt(D) * math.log2(math.e)
    r = np.einsum("bihd,bjhd->bhij", rh, kh)
    if causal:
        s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    mx = s.max(-1, keepdims=True)
    lse2 = (mx[..., 0] + np.log2(np.exp2(s - mx).sum(-1)))
    pr = np.exp2(s - lse2[..., None])
    rbar = (pr * np.where(np.isfinite(s), r, 0.0)).sum(-1)
    lrh = lr.double().cpu().numpy()
    assert np.abs(lrh[..., 0] - lse2).max() <= 2e-3 * max(1.0, np.abs(lse2).max())
    assert np.abs(lrh[..., 1] - rbar).max() <= 2e-2 * max(1.0, np.abs(rbar).max())
    ref = oracle.bwd(q.cpu(), k.cpu(), v.cpu(), rho.cpu(), dout.cpu(), causal=causal)
    _check(grads, ref, f"saved B{B} N{N} H{H} D{D} causal={causal} out={out_dtype}")
