"""parallax_decode_noalloc against parallax_decode, through the C ABI.

The allocation-free variant keeps the split records in the library's fixed
device scratch instead of a caller's workspace; it runs the same kernels, so
its output must equal parallax_decode's bit for bit (and therefore meet the
oracle's bar wherever parallax_decode does). Two calls in a row, the second
smaller, check that a call is not disturbed by what the previous one left
in the scratch.
"""

import pytest
import torch

import synth
import transformer_attention_parallax_amd as px
from gpu_helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(inp, splits, out_dtype=torch.float32, scale=None):
    ref = px.decode(inp["q"], inp["k"], inp["v"], inp["rho"], inp["seqlens"],
                    num_splits=splits, out_dtype=out_dtype, scale=scale)
    out = torch.full_like(ref, float("nan"))
    px.decode_noalloc(inp["q"], inp["k"], inp["v"], inp["rho"], inp["seqlens"],
                      out=out, num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_two_calls_second_smaller():
    big = synth.DecodeShape(B=2, H=16, D=128, L=8192, index=44)
    small = synth.DecodeShape(B=1, H=4, D=128, L=3000, index=45)
    announce("decode noalloc", "first call", big)
    inp = synth.decode_inputs(big, device=DEV)
    assert px.decode_splits(big.B, big.H, big.D, big.L) > 1
    ref, out = _both(inp, 0)
    assert torch.equal(out, ref)
    announce("decode noalloc", "second, smaller call", small)
    inp = synth.decode_inputs(small, device=DEV, ragged=True)
    ref, out = _both(inp, 5)
    assert torch.equal(out, ref)


@pytest.mark.parametrize("dtype,D,splits", [(torch.bfloat16, 64, 7), (torch.float32, 128, 3),
                                            (torch.float32, 64, 1)])
def test_noalloc_dtypes(dtype, D, splits):
    shp = synth.DecodeShape(B=3, H=2, D=D, L=1500, dtype=dtype, index=46)
    announce("decode noalloc dtypes", dtype, D, splits)
    inp = synth.decode_inputs(shp, device=DEV, ragged=True)
    for out_dtype in (torch.float32, torch.bfloat16):
        ref, out = _both(inp, splits, out_dtype=out_dtype, scale=-0.07)
        assert torch.equal(out, ref)


def test_noalloc_rejects_records_beyond_scratch():
    # 16 x 16 streams x 64 splits of 1040-byte records = 17 MB > 4 MiB: the
    # call fails on the host before any launch and leaves out untouched
    shp = synth.DecodeShape(B=16, H=16, D=128, L=4096, index=47)
    announce("decode noalloc oversize")
    assert px.decode_workspace_size(shp.B, shp.H, shp.D, shp.L, 64) > 4 << 20
    q = torch.zeros((shp.B, shp.H, shp.D), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((shp.B, shp.H, shp.L, shp.D), dtype=torch.bfloat16, device=DEV)
    out = torch.full((shp.B, shp.H, shp.D), 7.0, device=DEV)
    with pytest.raises(px.ParallaxError) as ei:
        px.decode_noalloc(q, kv, kv, q, out=out, num_splits=64)
    assert ei.value.status == px.ERR_WORKSPACE
    px.decode_noalloc(q, kv, kv, q, out=out, num_splits=1)  # no scratch needed
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
