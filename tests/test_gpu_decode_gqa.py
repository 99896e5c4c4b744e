"""GPU parity of parallax_decode_gqa (grouped query heads, contiguous or
paged KV cache) against the fp64 oracle, through the C ABI.

The oracle sees, for every query head, the keys and values of its kv head
in logical order (gathered from the pages on the host side of the test);
no new oracle arithmetic is involved. Tolerance 2e-2 (bf16 inputs, fp32
output), as for parallax_decode.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import transformer_attention_parallax_amd as px
from gpu_helpers import announce, max_abs_err, paginate as _paginate, poison_cache_tail

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2


def _make(B, Hq, Hkv, D, L, seed, ragged=True):
    g = synth.gen(seed, DEV)
    bf = lambda *s, sc=1.0: (sc * torch.randn(*s, device=DEV, generator=g)).to(torch.bfloat16)
    q, rho = bf(B, Hq, D), bf(B, Hq, D, sc=0.1)
    k, v = bf(B, Hkv, L, D), bf(B, Hkv, L, D)   # logical cache
    if ragged:
        lo = max(1, L // 3)
        sl = torch.randint(lo, L + 1, (B,), device=DEV, generator=g, dtype=torch.int32)
        sl[0] = L
    else:
        sl = torch.full((B,), L, dtype=torch.int32, device=DEV)
    return q, rho, k, v, sl


def _oracle(q, rho, k, v, sl, bh=None):
    """k, v: logical [B, Hkv, L, D]; expands kv heads to query heads."""
    B, Hq, D = q.shape
    G = Hq // k.shape[1]
    ke = k.repeat_interleave(G, dim=1)
    ve = v.repeat_interleave(G, dim=1)
    if bh is None:
        return oracle.decode(q.cpu(), rho.cpu(), ke.cpu(), ve.cpu(), seqlens=sl.cpu())
    out = []
    for b, h in bh:
        n = int(sl[b])
        out.append(oracle.decode(q[b:b + 1, h:h + 1].cpu(), rho[b:b + 1, h:h + 1].cpu(),
                                 ke[b:b + 1, h:h + 1, :n].cpu(), ve[b:b + 1, h:h + 1, :n].cpu(),
                                 seqlens=np.array([n], np.int32))[0, 0])
    return np.stack(out)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gqa_contiguous(G, D):
    B, Hkv, L = 3, 2, 700
    announce("gqa contiguous", G, D)
    q, rho, k, v, sl = _make(B, G * Hkv, Hkv, D, L, seed=900 + G + D)
    ref = _oracle(q, rho, k, v, sl)
    for splits in (0, 1, 3):
        out = px.decode_gqa(q, k, v, rho, seqlens=sl, num_splits=splits)
        torch.cuda.synchronize()
        err = max_abs_err(out, ref)
        assert err <= TOL, (splits, err)


@pytest.mark.parametrize("page", [16, 32, 64])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_gqa_paged(G, page):
    B, Hkv, L, D = 4, 2, 777, 128
    announce("gqa paged", G, page)
    q, rho, k, v, sl = _make(B, G * Hkv, Hkv, D, L, seed=920 + G + page)
    kp, vp, bt, npages = _paginate(k, v, page, seed=page + G)
    ref = _oracle(q, rho, k, v, sl)
    for splits in (0, 1, 5):
        out = px.decode_gqa(q, kp, vp, rho, seqlens=sl, block_table=bt, num_splits=splits)
        torch.cuda.synchronize()
        err = max_abs_err(out, ref)
        assert err <= TOL, (splits, err)
    ob = px.decode_gqa(q, kp, vp, rho, seqlens=sl, block_table=bt, out_dtype=torch.bfloat16)
    o32 = px.decode_gqa(q, kp, vp, rho, seqlens=sl, block_table=bt)
    torch.cuda.synchronize()
    assert torch.equal(ob, o32.to(torch.bfloat16))


@pytest.mark.parametrize("G,page", [(4, 16), (8, 32)])
def test_gqa_paged_head_major_pages(G, page):
    # pages stored [num_pages, Hkv, page, D] (each kv head's rows contiguous
    # in a page) and passed as the [num_pages, page, Hkv, D] view the entry
    # point takes: only the strides differ
    B, Hkv, L, D = 3, 2, 500, 128
    announce("gqa paged head-major", G, page)
    q, rho, k, v, sl = _make(B, G * Hkv, Hkv, D, L, seed=940 + G + page)
    kp, vp, bt, npages = _paginate(k, v, page, seed=page + 7 * G)
    kh = kp.transpose(1, 2).contiguous().transpose(1, 2)
    vh = vp.transpose(1, 2).contiguous().transpose(1, 2)
    assert kh.stride(1) == D and kh.stride(2) == page * D
    ref = _oracle(q, rho, k, v, sl)
    for splits in (0, 1, 4):
        out = px.decode_gqa(q, kh, vh, rho, seqlens=sl, block_table=bt, num_splits=splits)
        torch.cuda.synchronize()
        err = max_abs_err(out, ref)
        assert err <= TOL, (splits, err)


def test_gqa_paged_skips_invalid_pages():
    """A page index outside [0, num_pages) removes that page's keys."""
    B, G, Hkv, L, D, page = 2, 4, 2, 256, 64, 32
    announce("gqa invalid pages")
    q, rho, k, v, _ = _make(B, G * Hkv, Hkv, D, L, seed=940, ragged=False)
    sl = torch.full((B,), L, dtype=torch.int32, device=DEV)
    kp, vp, bt, npages = _paginate(k, v, page, seed=7)
    bt[1, 2] = npages + 5      # keys 64..95 of sequence 1 are skipped
    bt[0, 5] = -3              # keys 160..191 of sequence 0 are skipped
    out = px.decode_gqa(q, kp, vp, rho, seqlens=sl, block_table=bt)
    torch.cuda.synchronize()
    keep = [torch.cat([torch.arange(0, 160), torch.arange(192, L)]),
            torch.cat([torch.arange(0, 64), torch.arange(96, L)])]
    for b in range(B):
        kb, vb = k[b:b + 1, :, keep[b].to(DEV)], v[b:b + 1, :, keep[b].to(DEV)]
        n = torch.tensor([kb.shape[2]], dtype=torch.int32, device=DEV)
        ref = _oracle(q[b:b + 1], rho[b:b + 1], kb, vb, n)
        assert max_abs_err(out[b:b + 1], ref) <= TOL


def test_gqa_group1_matches_mha_decode():
    """G = 1 is parallax_decode. The grouped kernel feeds the weights p and
    p r to the matrix cores as hi + lo bf16 pairs (relative error < 2^-16
    per weight, l and A_r summed from the same pairs); the MHA kernel keeps
    them in fp32 and sums in another order. Outputs are weighted means of
    values of size ~4."""
    B, H, L, D = 2, 4, 1000, 128
    announce("gqa G=1 vs decode")
    q, rho, k, v, sl = _make(B, H, H, D, L, seed=950)
    a = px.decode_gqa(q, k, v, rho, seqlens=sl)
    b = px.decode(q, k, v, rho, sl)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(a - b)).item() <= 1e-4
    assert max_abs_err(a, _oracle(q, rho, k, v, sl)) <= TOL


def test_gqa_paged_large_sampled():
    """256 sequences x 32 query heads / 8 kv heads x 8192 context, 16-token
    pages in shuffled order: sampled (b, head) rows against the oracle."""
    B, Hq, Hkv, L, D, page = 256, 32, 8, 8192, 128, 16
    announce("gqa paged large")
    g = synth.gen(960, DEV)
    npb = L // page
    num_pages = B * npb
    perm = torch.randperm(num_pages, generator=torch.Generator().manual_seed(3))
    bt = perm.view(B, npb).to(torch.int32).to(DEV)
    kp = torch.randn(num_pages, page, Hkv, D, device=DEV, generator=g).to(torch.bfloat16)
    vp = torch.randn(num_pages, page, Hkv, D, device=DEV, generator=g).to(torch.bfloat16)
    q = torch.randn(B, Hq, D, device=DEV, generator=g).to(torch.bfloat16)
    rho = (0.1 * torch.randn(B, Hq, D, device=DEV, generator=g)).to(torch.bfloat16)
    sl = torch.full((B,), L, dtype=torch.int32, device=DEV)
    out = px.decode_gqa(q, kp, vp, rho, seqlens=sl, block_table=bt)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    G = Hq // Hkv
    for b, h in [(0, 0), (17, 31), (128, 9), (255, 20)]:
        pages = bt[b].long()
        kl = kp[pages][:, :, h // G].reshape(L, D)
        vl = vp[pages][:, :, h // G].reshape(L, D)
        ref = oracle.decode(q[b:b + 1, h:h + 1].cpu(), rho[b:b + 1, h:h + 1].cpu(),
                            kl.view(1, 1, L, D).cpu(), vl.view(1, 1, L, D).cpu())
        assert max_abs_err(out[b:b + 1, h:h + 1], ref) <= TOL, (b, h)
    del kp, vp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("paged", [False, True])
def test_gqa_single_key_returns_v(paged):
    """One visible key: p = 1, l = 1 and the covariance term vanishes, so the
    output is that key's value exactly (the weight 1 and r are exact in bf16
    products, and vbar*rbar and A_rv/l round identically)."""
    B, G, Hkv, L, D = 3, 4, 2, 64, 128
    announce("gqa single key", paged)
    q, rho, k, v, _ = _make(B, G * Hkv, Hkv, D, L, seed=970, ragged=False)
    sl = torch.tensor([1, 1, 0], dtype=torch.int32, device=DEV)
    if paged:
        kp, vp, bt, _ = _paginate(k, v, 16, seed=11)
        out = px.decode_gqa(q, kp, vp, rho, seqlens=sl, block_table=bt)
    else:
        out = px.decode_gqa(q, k, v, rho, seqlens=sl)
    torch.cuda.synchronize()
    ref = v[:, :, 0].float().repeat_interleave(G, dim=1)
    assert torch.equal(out[:2], ref[:2])
    assert torch.equal(out[2], torch.zeros_like(out[2]))     # empty sequence


@pytest.mark.parametrize("D,page", [(128, 16), (64, 8), (128, 8)])
def test_gqa_masked_rows_hold_nan(D, page):
    """Rows past each sequence's length in its last page, the spare pages and
    page 0 (where skipped pages are redirected) hold NaN; none may leak."""
    B, G, Hkv, L = 3, 8, 2, 300
    announce("gqa NaN in masked rows", D, page)
    q, rho, k, v, sl = _make(B, G * Hkv, Hkv, D, L, seed=971)
    npb = (L + page - 1) // page
    num_pages = 1 + B * npb + 2
    kp = torch.full((num_pages, page, Hkv, D), float("nan"), device=DEV).to(torch.bfloat16)
    vp = kp.clone()
    perm = 1 + torch.randperm(num_pages - 1, generator=torch.Generator().manual_seed(5))
    bt = perm[: B * npb].view(B, npb).to(torch.int32)
    for b in range(B):
        n = int(sl[b])
        for j in range((n + page - 1) // page):
            t = min(page, n - j * page)
            kp[bt[b, j], :t] = k[b, :, j * page: j * page + t].permute(1, 0, 2)
            vp[bt[b, j], :t] = v[b, :, j * page: j * page + t].permute(1, 0, 2)
    bt[0, 1] = -1                         # keys page..2*page-1 of sequence 0 skipped
    bt = bt.to(DEV)
    out = px.decode_gqa(q, kp, vp, rho, seqlens=sl, block_table=bt)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    for b in range(B):
        n = int(sl[b])
        keep = torch.arange(n)
        if b == 0:
            keep = keep[(keep < page) | (keep >= 2 * page)]
        kb, vb = k[b:b + 1, :, keep.to(DEV)], v[b:b + 1, :, keep.to(DEV)]
        m = torch.tensor([kb.shape[2]], dtype=torch.int32, device=DEV)
        ref = _oracle(q[b:b + 1], rho[b:b + 1], kb, vb, m)
        assert max_abs_err(out[b:b + 1], ref) <= TOL, b


def test_gqa_growing_logits_rescale():
    """Keys aligned with q and growing along the sequence: the running max
    moves by more than the lazy-rescale headroom again and again."""
    B, G, Hkv, L, D = 2, 4, 2, 1500, 128
    announce("gqa growing logits")
    q, rho, k, v, sl = _make(B, G * Hkv, Hkv, D, L, seed=972, ragged=False)
    qa = q.float().view(B, Hkv, G, D).mean(dim=2)           # shared direction per kv head
    ramp = torch.linspace(0.0, 6.0, L, device=DEV).view(1, 1, L, 1)
    k = (0.3 * k.float() + ramp * qa.unsqueeze(2) / qa.norm(dim=-1, keepdim=True).unsqueeze(2)
         * 12.0).to(torch.bfloat16)
    for scale in (None, 0.5):
        out = px.decode_gqa(q, k, v, rho, seqlens=sl, scale=scale)
        torch.cuda.synchronize()
        ref = oracle.decode(q.cpu(), rho.cpu(), k.repeat_interleave(G, 1).cpu(),
                            v.repeat_interleave(G, 1).cpu(), seqlens=sl.cpu(),
                            scale=scale if scale is not None else 1.0 / D ** 0.5)
        assert max_abs_err(out, ref) <= TOL, scale


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_gqa_negative_and_zero_scale(scale):
    B, G, Hkv, L, D = 2, 2, 2, 333, 64
    announce("gqa scale", scale)
    q, rho, k, v, sl = _make(B, G * Hkv, Hkv, D, L, seed=973)
    kp, vp, bt, _ = _paginate(k, v, 32, seed=12)
    out = px.decode_gqa(q, kp, vp, rho, seqlens=sl, block_table=bt, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.decode(q.cpu(), rho.cpu(), k.repeat_interleave(G, 1).cpu(),
                        v.repeat_interleave(G, 1).cpu(), seqlens=sl.cpu(), scale=scale)
    assert max_abs_err(out, ref) <= TOL


GROUPED_MIN_KEYS = 1 << 17   # paged: sequences x kv-head groups x cache length


def _grouped_len(B, Hkv, paged):
    """Cache length that puts a batch of B sequences in workgroups of
    several kv heads: paged caches with groups of at least 4 kv heads from
    2^17 keys of work, contiguous ones once B x kv-head groups reaches
    256 * 8 / heads per workgroup."""
    nh = 8
    while Hkv % nh:
        nh //= 2
    if paged:
        assert nh >= 4
    else:
        assert B * (Hkv // nh) >= 256 * 8 // nh
        return 1024
    L = -(-GROUPED_MIN_KEYS // (B * (Hkv // nh)))
    return max(1024, -(-L // 64) * 64)


@pytest.mark.parametrize("G,Hkv,D,B,paged", [
    (4, 12, 128, 6, True), (1, 8, 64, 4, True), (8, 4, 128, 5, True), (2, 8, 128, 300, True),
    (4, 2, 128, 1024, False), (8, 4, 64, 512, False), (2, 8, 128, 300, False)])
def test_gqa_grouped_workgroups(G, Hkv, D, B, paged):
    """The workgroup shape the library takes for large enough batches: one
    wave per kv head, up to 8 kv heads of a sequence per workgroup, walking
    the same tiles in step (split for the paged batches of 4 to 8
    sequences, unsplit for the rest). The cache holds one full-length
    sequence and short ragged ones (one empty, one of a single key), with
    NaN in every row past a sequence's end; sampled (b, query head) streams
    are compared with the oracle, planned and explicit split counts agree,
    the empty sequence gives zeros and a bf16 output is the RNE rounding of
    the fp32 one."""
    L = _grouped_len(B, Hkv, paged)
    announce("gqa grouped", G, Hkv, D, B, L, "paged" if paged else "contiguous")
    q, rho, k, v, _ = _make(B, G * Hkv, Hkv, D, L, seed=990 + G + Hkv + D + B, ragged=False)
    g = torch.Generator().manual_seed(991 + B)
    sl = torch.randint(2, 700, (B,), generator=g, dtype=torch.int32)
    sl[0], sl[1], sl[2 % B] = L, 0, 1
    sl = sl.to(DEV)
    poison_cache_tail(k, sl)            # rows past each sequence hold NaN
    poison_cache_tail(v, sl)
    if paged:
        kc, vc, bt, _ = _paginate(k, v, 16, seed=992 + B)
        kw = dict(block_table=bt)
    else:
        kc, vc, kw = k, v, {}
    # the full-length sequence: its first and last query head; sequences
    # 1..3: every query head; then every (B // 16)-th sequence, two heads
    bh = [(0, 0), (0, G * Hkv - 1)]
    bh += [(b, h) for b in range(1, min(B, 4)) for h in range(G * Hkv)]
    bh += [(b, h) for b in range(4, B, max(1, B // 16)) for h in (0, G * Hkv - 1)]
    ref = _oracle(q, rho, k, v, sl, bh=bh)
    outs = []
    for splits in (0, 1, 7):
        out = px.decode_gqa(q, kc, vc, rho, seqlens=sl, num_splits=splits, **kw)
        torch.cuda.synchronize()
        got = torch.stack([out[b, h] for b, h in bh])
        err = max_abs_err(got, ref)
        assert err <= TOL, (splits, err)
        assert torch.count_nonzero(out[1]).item() == 0
        outs.append(out)
    assert max_abs_err(outs[0], outs[1].cpu().double().numpy()) <= 1e-4
    ob = px.decode_gqa(q, kc, vc, rho, seqlens=sl, out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    assert torch.equal(ob, outs[0].to(torch.bfloat16))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,splits", [(1, 9), (2, 2), (8, 40)])
def test_gqa_split_workspace_garbage_and_reuse(G, splits, D):
    """Split grouped-query decode with a NaN-filled workspace reused by
    repeated calls: bit-identical outputs within the oracle's bar; a bf16
    output is the RNE rounding of the fp32 one."""
    B, Hkv, L = 3, 2, 6000
    announce("gqa split workspace", G, splits, D)
    q, rho, k, v, sl = _make(B, G * Hkv, Hkv, D, L, seed=960 + G + D + splits)
    need = px.decode_gqa_workspace_size(B, G * Hkv, Hkv, D, L, splits)
    ws = torch.full((need // 4 + 16,), float("nan"), device=DEV).view(torch.uint8)
    outs = []
    for _ in range(3):
        outs.append(px.decode_gqa(q, k, v, rho, seqlens=sl, num_splits=splits, workspace=ws))
        torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    assert max_abs_err(outs[0], _oracle(q, rho, k, v, sl)) <= TOL
    ob = px.decode_gqa(q, k, v, rho, seqlens=sl, num_splits=splits, workspace=ws,
                       out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(ob, outs[0].to(torch.bfloat16))
