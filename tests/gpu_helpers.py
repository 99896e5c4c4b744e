"""Helpers for the GPU parity tests (inputs from synth, expectations from the
oracle; nothing here computes attention)."""

from __future__ import annotations

import sys

import numpy as np
import torch

TOL_F32 = 1e-4   # max abs error, fp32 inputs
TOL_BF16 = 2e-2  # max abs error, bf16 inputs (fp32 accumulation, fp32 out)


def tol_for(dtype) -> float:
    return TOL_BF16 if dtype == torch.bfloat16 else TOL_F32


def announce(*parts):
    """Name the case on stdout before a GPU step (flushed)."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def max_abs_err(gpu: torch.Tensor, ref: np.ndarray) -> float:
    g = gpu.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return float(np.max(np.abs(g - ref))) if g.size else 0.0


def poison_cache_tail(cache: torch.Tensor, seqlens: torch.Tensor):
    """Fill positions at or beyond each sequence length with NaN."""
    lens = seqlens.cpu().tolist()
    for b, n in enumerate(lens):
        if n < cache.shape[2]:
            cache[b, :, max(n, 0):] = float("nan")


def paginate(k, v, page, seed, spare=3):
    """Scatter logical [B, Hkv, L, D] caches into shuffled pages
    [num_pages, page, Hkv, D]; returns caches and the int32 block table."""
    B, Hkv, L, D = k.shape
    npb = (L + page - 1) // page
    num_pages = B * npb + spare
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(num_pages, generator=g)[: B * npb].view(B, npb).to(torch.int32)
    kp = torch.full((num_pages, page, Hkv, D), float("nan"), device=k.device).to(torch.bfloat16)
    vp = kp.clone()
    pad = npb * page - L
    kl = torch.nn.functional.pad(k, (0, 0, 0, pad)).view(B, Hkv, npb, page, D)
    vl = torch.nn.functional.pad(v, (0, 0, 0, pad)).view(B, Hkv, npb, page, D)
    for b in range(B):
        idx = perm[b].long().to(k.device)
        kp[idx] = kl[b].permute(1, 2, 0, 3)
        vp[idx] = vl[b].permute(1, 2, 0, 3)
    return kp, vp, perm.to(k.device), num_pages
