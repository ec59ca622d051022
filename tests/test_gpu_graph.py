"""The two calls under HIP graph capture (the page's CUDA-graph requirement:
the fused kernel must be capturable).  The library allocates nothing, never
synchronises and records no memset, so a captured build + attention pair must
replay to the eager result, and follow in-place input updates."""

import pytest
import torch

from relative_position_bias_relpos_amd import binding as rp
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _buffers(d):
    g = G.to_dev(d)
    H, W = d["H"], d["W"]
    shp = g["q"].shape
    g["rel_h"] = torch.empty(shp[:3] + (H,), dtype=torch.float32, device="cuda")
    g["rel_w"] = torch.empty(shp[:3] + (W,), dtype=torch.float32, device="cuda")
    g["out"] = torch.empty(shp, dtype=torch.float32, device="cuda")
    return g


def _run(g, d):
    rp.relpos_build(g["q"], g["rel_pos_h"], g["rel_pos_w"], d["H"], d["W"], rel_h=g["rel_h"], rel_w=g["rel_w"])
    rp.relpos_attn_fwd(g["q"], g["k"], g["v"], g["rel_h"], g["rel_w"], d["H"], d["W"], d["scale"], out=g["out"])


@pytest.mark.parametrize("name,kw", [("rect", dict(B=1, heads=2, H=24, W=40)), ("deepencoder", {})])
def test_graph_replays_match_eager(name, kw):
    d = G.make(name, **kw)
    g = _buffers(d)
    _run(g, d)
    torch.cuda.synchronize()
    ref = g["out"].clone()

    # warm up on a side stream, as torch's capture recipe does
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _run(g, d)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run(g, d)
    torch.cuda.synchronize()

    for i in range(4):
        g["out"].fill_(float("nan"))
        g["rel_h"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g["out"], ref), (name, i)
        # unrelated eager work between replays
        x = torch.randn(1 << 20, device="cuda")
        (x * 2).sum().item()

    # in-place input update: the replay follows it and matches eager on new data
    d2 = G.make(name, seed=7, **kw)
    for key in ("q", "k", "v", "rel_pos_h", "rel_pos_w"):
        g[key].copy_(d2[key].cuda())
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    got = g["out"].clone()
    _run(g, d)
    torch.cuda.synchronize()
    assert torch.equal(got, g["out"]), name
    assert not torch.equal(got, ref), name


@pytest.mark.parametrize("name,kw", [("rect", dict(B=1, heads=3, H=21, W=35)), ("deepencoder", {})])
def test_fused_graph_replays_match_eager(name, kw):
    """relpos_attn_fused with a caller workspace under capture: the persistent
    kernel and the merge replay to the eager result and follow input updates."""
    d = G.make(name, **kw)
    g = _buffers(d)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B, nh = g["q"].shape[:2]
    ws = torch.empty(rp.fused_workspace_bytes(B, nh, d["H"], d["W"], g["q"].dtype, cus), dtype=torch.uint8,
                     device="cuda")

    def run():
        rp.relpos_attn_fused(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], d["H"], d["W"], d["scale"],
                             out=g["out"], workspace=ws)

    run()
    torch.cuda.synchronize()
    ref = g["out"].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for i in range(4):
        g["out"].fill_(float("nan"))
        ws.fill_(0xff)  # the workspace is scratch: stale contents must not matter
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g["out"], ref), (name, i)
        x = torch.randn(1 << 20, device="cuda")
        (x * 2).sum().item()
    d2 = G.make(name, seed=7, **kw)
    for key in ("q", "k", "v", "rel_pos_h", "rel_pos_w"):
        g[key].copy_(d2[key].cuda())
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    got = g["out"].clone()
    run()
    torch.cuda.synchronize()
    assert torch.equal(got, g["out"]), name
    assert not torch.equal(got, ref), name
