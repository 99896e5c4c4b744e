"""Decode captured in a HIP graph (torch.cuda.graph) and replayed.

Serving loops capture a decode step once and replay it with new inputs in
the same buffers. Both decode entry points are captured with a context long
enough to be split (split kernel plus combine launch); between replays the
query and probe are rewritten in place by ordinary eager work, and every
replay must equal an eager call on the same inputs bit for bit (the graph
runs the same kernels). The library records no memory fills, so nothing in
the graph depends on a fill node.
"""

import pytest
import torch

import synth
import transformer_attention_parallax_amd as px
from gpu_helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_graph_replays(noalloc):
    shp = synth.DecodeShape(B=2, H=16, D=128, L=4096, index=60)
    announce("decode graph capture", "noalloc" if noalloc else "workspace", shp)
    inp = synth.decode_inputs(shp, device=DEV)
    assert px.decode_splits(shp.B, shp.H, shp.D, shp.L) > 1
    q, rho = inp["q"].clone(), inp["rho"].clone()
    out = torch.empty((shp.B, shp.H, shp.D), device=DEV)
    ws = None
    if not noalloc:
        ws = torch.empty(px.decode_workspace_size(shp.B, shp.H, shp.D, shp.L),
                         dtype=torch.uint8, device=DEV)

    def step():
        if noalloc:
            px.decode_noalloc(q, inp["k"], inp["v"], rho, inp["seqlens"], out=out)
        else:
            px.decode(q, inp["k"], inp["v"], rho, inp["seqlens"], out=out, workspace=ws)

    # warm up on a side stream (also fixes the scratch address before capture)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    g = synth.gen(61, DEV)
    for i in range(5):
        # eager work between replays: new query and probe in the captured buffers
        q.copy_(torch.randn(q.shape, device=DEV, generator=g).to(q.dtype))
        rho.copy_((0.1 * torch.randn(rho.shape, device=DEV, generator=g)).to(rho.dtype))
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        ref = px.decode(q, inp["k"], inp["v"], rho, inp["seqlens"])
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
