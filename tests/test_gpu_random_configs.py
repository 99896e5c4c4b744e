"""Seeded random configurations of every entry point against the fp64 oracle.

Each case draws its sizes, layout, lengths, split count and scale from a
numpy generator seeded by the case number (sizes only; the tensors come from
``synth``), so a failure names a configuration that can be rebuilt exactly.
The configurations mix what the fixed-shape tests take one at a time: odd
head counts, ragged and empty sequences, strided input and output views,
requested split counts, negative scales, and both workgroup shapes of the
grouped-query kernel. Bars are those of the fixed-shape tests: max abs
error 1e-4 (fp32 inputs) or 2e-2 (bf16 inputs) for the outputs, 1e-2 of
the largest reference entry for the gradients.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import transformer_attention_parallax_amd as px
from gpu_helpers import announce, max_abs_err, paginate, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_BF16 = 2e-2

# sequences x kv-head groups x cache length at which a paged cache takes the
# grouped workgroup shape (one wave per kv head)
GROUPED_MIN_KEYS = 1 << 17


def _cfg_rng(tag, case):
    return np.random.default_rng([tag, case])


def _scale(rng, D):
    u = rng.random()
    if u < 0.5:
        return None
    if u < 0.7:
        return -float(rng.uniform(0.05, 0.2))
    return float(rng.uniform(0.02, 0.25))


def _lengths(rng, B, L):
    sl = rng.integers(0, L + 1, size=B)
    sl[rng.integers(0, B)] = L
    if B > 2 and rng.random() < 0.5:
        sl[rng.integers(0, B)] = 0
    return torch.tensor(sl, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("case", range(24))
def test_random_decode(case):
    rng = _cfg_rng(1, case)
    B, H = int(rng.integers(1, 7)), int(rng.integers(1, 6))
    D = int(rng.choice([64, 128]))
    L = int(rng.integers(1, 1600))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    splits = int(rng.choice([0, 0, 1, int(rng.integers(2, 40))]))
    token_major = bool(rng.random() < 0.5)
    scale = _scale(rng, D)
    use_rho = bool(rng.random() < 0.85)
    announce("random decode", case, B, H, D, L, dtype, splits, token_major, scale, use_rho)

    g = synth.gen(3000 + case, DEV)
    mk = lambda *s, sc=1.0: (sc * torch.randn(*s, device=DEV, generator=g)).to(dtype)
    qr = mk(B, H, 2 * D)                     # q and rho as strided halves of one buffer
    qr[..., D:] = (0.1 * qr[..., D:].float()).to(dtype)
    q = qr[..., :D]
    rho = qr[..., D:] if use_rho else None
    if token_major:                          # cache stored [B, L, H, D]
        k = mk(B, L, H, D).permute(0, 2, 1, 3)
        v = mk(B, L, H, D).permute(0, 2, 1, 3)
    else:
        k, v = mk(B, H, L, D), mk(B, H, L, D)
    sl = _lengths(rng, B, L)
    strided_out = bool(rng.random() < 0.5)   # out as the upper half of [B, H, 2D]

    big = torch.zeros(B, H, 2 * D, device=DEV)
    out = px.decode(q, k, v, rho, sl, scale=scale, num_splits=splits,
                    out=big[..., D:] if strided_out else None)
    ob = px.decode(q, k, v, rho, sl, scale=scale, num_splits=splits,
                   out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.count_nonzero(big[..., :D]).item() == 0
    rz = torch.zeros_like(q) if rho is None else rho
    ref = oracle.decode(q.cpu(), rz.cpu(), k.contiguous().cpu(), v.contiguous().cpu(),
                        seqlens=sl.cpu(), scale=scale)
    err = max_abs_err(out, ref)
    print(f"decode case {case}: err {err:.3e}", flush=True)
    assert err <= tol_for(dtype), (case, err)
    assert torch.equal(ob, out.to(torch.bfloat16))


@pytest.mark.parametrize("case", range(20))
def test_random_decode_gqa(case):
    rng = _cfg_rng(2, case)
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    paged = bool(rng.random() < 0.6)
    grouped = bool(rng.random() < 0.4)
    page = int(rng.choice([8, 16, 32, 64])) if paged else 0
    if grouped and paged:
        # groups of 4 or 8 kv heads, enough keys for the grouped shape
        Hkv = int(rng.choice([4, 8, 12]))
        B = int(rng.integers(1, 4))
        L = -(-GROUPED_MIN_KEYS // B) + int(rng.integers(0, 3000))
    elif grouped:
        # contiguous caches take it when every sequence's kv heads fill the chip
        Hkv, B, L = 8, int(rng.integers(256, 300)), int(rng.integers(1, 200))
    else:
        Hkv, B, L = int(rng.integers(1, 5)), int(rng.integers(1, 5)), int(rng.integers(1, 1200))
    splits = int(rng.choice([0, 0, 1, int(rng.integers(2, 12))]))
    scale = _scale(rng, D)
    Hq = G * Hkv
    announce("random gqa", case, B, Hq, Hkv, D, L, paged, page, grouped, splits, scale)

    g = synth.gen(3100 + case, DEV)
    bf = lambda *s, sc=1.0: (sc * torch.randn(*s, device=DEV, generator=g)).to(torch.bfloat16)
    q, rho = bf(B, Hq, D), bf(B, Hq, D, sc=0.1)
    k, v = bf(B, Hkv, L, D), bf(B, Hkv, L, D)
    sl = _lengths(rng, B, L)
    strided = bool(rng.random() < 0.5)   # q, rho halves of one buffer; out a strided view
    big = torch.zeros(B, Hq, 2 * D, device=DEV)
    if strided:
        qr = torch.cat([q, rho], dim=-1)
        q, rho = qr[..., :D], qr[..., D:]
    kw = dict(seqlens=sl, scale=scale, num_splits=splits)
    if paged:
        kp, vp, bt, _ = paginate(k, v, page, seed=case)
        out = px.decode_gqa(q, kp, vp, rho, block_table=bt,
                            out=big[..., D:] if strided else None, **kw)
        ob = px.decode_gqa(q, kp, vp, rho, block_table=bt, out_dtype=torch.bfloat16, **kw)
        del kp, vp
    else:
        out = px.decode_gqa(q, k, v, rho, out=big[..., D:] if strided else None, **kw)
        ob = px.decode_gqa(q, k, v, rho, out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    assert torch.equal(ob, out.to(torch.bfloat16))
    assert torch.count_nonzero(big[..., :D]).item() == 0
    # the oracle sees each query head's kv head in logical order; large
    # cases are checked on sampled (sequence, head) rows
    if B * Hq <= 256 and B * Hq * L <= 4_000_000:
        ref = oracle.decode(q.cpu(), rho.cpu(), k.repeat_interleave(G, 1).cpu(),
                            v.repeat_interleave(G, 1).cpu(), seqlens=sl.cpu(), scale=scale)
        err = max_abs_err(out, ref)
    else:
        pairs = {(int(rng.integers(0, B)), int(rng.integers(0, Hq))) for _ in range(10)}
        pairs = sorted(pairs | {(0, 0), (B - 1, Hq - 1)})
        qc, rc, slc = q.cpu(), rho.cpu(), sl.cpu()
        refs = []
        for b, h in pairs:
            n = int(slc[b])
            refs.append(oracle.decode(qc[b:b + 1, h:h + 1], rc[b:b + 1, h:h + 1],
                                      k[b:b + 1, h // G:h // G + 1, :max(n, 1)].cpu(),
                                      v[b:b + 1, h // G:h // G + 1, :max(n, 1)].cpu(),
                                      seqlens=np.array([n], np.int32), scale=scale)[0, 0])
        got = torch.stack([out[b, h] for b, h in pairs])
        err = max_abs_err(got, np.stack(refs))
    print(f"gqa case {case}: err {err:.3e}", flush=True)
    assert err <= TOL_BF16, (case, err)
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("case", range(16))
def test_random_prefill(case):
    rng = _cfg_rng(3, case)
    B, N, H = int(rng.integers(1, 3)), int(rng.integers(1, 220)), int(rng.integers(1, 4))
    D = int(rng.choice([64, 128]))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    causal = bool(rng.random() < 0.7)
    fused = bool(rng.random() < 0.5)
    scale = _scale(rng, D)
    announce("random prefill", case, B, N, H, D, dtype, causal, fused, scale)

    g = synth.gen(3200 + case, DEV)
    mk = lambda *s, sc=1.0: (sc * torch.randn(*s, device=DEV, generator=g)).to(dtype)
    if fused:                                # q, k, v, rho as views of one [B, N, 4, H, D]
        t = mk(B, N, 4, H, D)
        t[:, :, 3] = (0.1 * t[:, :, 3].float()).to(dtype)
        q, k, v, rho = t.unbind(2)
    else:
        q, k, v, rho = mk(B, N, H, D), mk(B, N, H, D), mk(B, N, H, D), mk(B, N, H, D, sc=0.1)
    out = px.fwd(q, k, v, rho, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.fwd(q.cpu(), k.cpu(), v.cpu(), rho.cpu(), scale=scale, causal=causal)
    err = max_abs_err(out, ref)
    print(f"prefill case {case}: err {err:.3e}", flush=True)
    assert err <= tol_for(dtype), (case, err)


@pytest.mark.parametrize("case", range(10))
def test_random_varlen(case):
    rng = _cfg_rng(4, case)
    nseq = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.integers(0, 320, size=nseq)]
    if rng.random() < 0.3:
        lens[int(rng.integers(0, nseq))] = 0
    H, D = int(rng.integers(1, 4)), int(rng.choice([64, 128]))
    causal = bool(rng.random() < 0.7)
    scale = _scale(rng, D)
    lead, tail = int(rng.integers(0, 5)), int(rng.integers(0, 5))
    announce("random varlen", case, lens, H, D, causal, scale, lead, tail)

    g = synth.gen(3300 + case, DEV)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64) + lead
    T = int(cu[-1]) + tail
    mk = lambda s=1.0: (s * torch.randn(T, H, D, device=DEV, generator=g)).to(torch.bfloat16)
    q, k, v, rho = mk(), mk(), mk(), mk(0.1)
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    max_len = max(lens) + int(rng.integers(0, 40))     # an upper bound, not always tight
    out = torch.full((T, H, D), float("nan"), device=DEV)
    px.fwd_varlen(q, k, v, rho, cu_t, max_len, causal=causal, scale=scale, out=out)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        rows = slice(int(cu[b]), int(cu[b]) + L)
        if L:
            ref = oracle.fwd(*(t[rows].unsqueeze(0).cpu() for t in (q, k, v, rho)),
                             scale=scale, causal=causal)
            err = max_abs_err(out[rows].unsqueeze(0), ref)
            assert err <= TOL_BF16, (case, b, L, err)
    if lead:
        assert torch.isnan(out[:lead]).all().item()
    if tail:
        assert torch.isnan(out[T - tail:]).all().item()


def _check_grads(grads, ref, what):
    for name, a, r in zip(("dq", "dk", "dv", "drho"), grads, ref):
        a = a.double().cpu().numpy()
        assert np.isfinite(a).all(), f"{what} {name}: non-finite"
        err = float(np.abs(a - r).max())
        bound = 1e-2 * float(np.abs(r).max()) + 1e-5
        print(f"{what} {name}: err {err:.3e} bound {bound:.3e}", flush=True)
        assert err <= bound, (what, name, err, bound)


@pytest.mark.parametrize("case", range(10))
def test_random_backward(case):
    rng = _cfg_rng(5, case)
    B, N, H = int(rng.integers(1, 3)), int(rng.integers(1, 160)), int(rng.integers(1, 3))
    D = int(rng.choice([64, 128]))
    causal = bool(rng.random() < 0.7)
    scale = _scale(rng, D)
    rho_std = float(rng.choice([0.0, 0.1, 0.3]))
    saved = bool(rng.random() < 0.5)
    announce("random backward", case, B, N, H, D, causal, scale, rho_std, saved)

    g = synth.gen(3400 + case, DEV)
    mk = lambda s=1.0: (s * torch.randn(B, N, H, D, device=DEV, generator=g)).to(torch.bfloat16)
    q, k, v, rho, dout = mk(), mk(), mk(), mk(rho_std), mk()
    if saved:
        out, vbar, lse_rbar = px.fwd_train(q, k, v, rho, causal=causal, scale=scale)
        grads = px.bwd_saved(q, k, v, rho, dout, out, vbar, lse_rbar, causal=causal,
                             scale=scale)
    else:
        grads = px.bwd(q, k, v, rho, dout, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.bwd(q.cpu(), k.cpu(), v.cpu(), rho.cpu(), dout.cpu(), scale=scale,
                     causal=causal)
    _check_grads(grads, ref, f"backward case {case}")
