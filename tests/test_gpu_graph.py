"""The calls under HIP graph capture and across streams (the page's
CUDA-graph requirement: the fused kernel must be capturable).  The library
allocates nothing, never synchronises and records no memset, so a captured
build + attention pair (or fused call) must replay to the oracle's result and
to the eager one, and follow in-place input updates; and calls enqueued on a
side stream must order correctly against producers and consumers on others."""

import numpy as np
import pytest
import torch

from relative_position_bias_relpos_amd import binding as rp
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _vs_oracle(tag, got, d):
    ref, _, _ = G.oracle_full(d)
    err = np.abs(G.f64(got) - ref)
    print(f"[graph] {tag}: n={err.size} max={err.max():.3e} mean={err.mean():.3e}", flush=True)
    assert np.isfinite(err).all(), tag
    assert err.max() <= G.MAX_ABS, tag
    assert err.mean() <= G.MEAN_ABS, tag


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
        if i == 0 and name == "rect":
            _vs_oracle(f"{name} replay", g["out"], d)
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
    if name == "rect":
        _vs_oracle(f"{name} replay after the seed-7 update", got, d2)
    _run(g, d)
    torch.cuda.synchronize()
    assert torch.equal(got, g["out"]), name
    assert not torch.equal(got, ref), name


@pytest.mark.parametrize("name,kw", [("rect", dict(B=1, heads=3, H=21, W=35)), ("deepencoder", {}),
                                     ("tiny", dict(B=2, heads=3, H=14, W=14))])
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
        if i == 0 and name == "rect":
            _vs_oracle(f"fused {name} replay", g["out"], d)
        x = torch.randn(1 << 20, device="cuda")
        (x * 2).sum().item()
    d2 = G.make(name, seed=7, **kw)
    for key in ("q", "k", "v", "rel_pos_h", "rel_pos_w"):
        g[key].copy_(d2[key].cuda())
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    got = g["out"].clone()
    if name == "rect":
        _vs_oracle(f"fused {name} replay after the seed-7 update", got, d2)
    run()
    torch.cuda.synchronize()
    assert torch.equal(got, g["out"]), name
    assert not torch.equal(got, ref), name


@pytest.mark.parametrize("path", ["two-call", "fused"])
def test_stream_ordering(path):
    """Inputs produced by a kernel on stream A (behind an event), both library
    calls enqueued on stream B, the output consumed by a kernel on stream C
    after an event recorded on B; nothing synchronises the host in between.
    The consumer's copy must equal the oracle's result."""
    d = G.make("rect", B=1, heads=3, H=24, W=40)
    host = {key: d[key].pin_memory() for key in ("q", "k", "v", "rel_pos_h", "rel_pos_w")}
    H, W = d["H"], d["W"]
    sa, sb, sc = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    dev = {key: torch.empty_like(t, device="cuda") for key, t in host.items()}
    rel_h = torch.empty(dev["q"].shape[:3] + (H,), dtype=torch.float32, device="cuda")
    rel_w = torch.empty(dev["q"].shape[:3] + (W,), dtype=torch.float32, device="cuda")
    out = torch.empty(dev["q"].shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(rp.fused_workspace_bytes(1, 3, H, W, dev["q"].dtype, G.cu_count()), dtype=torch.uint8,
                     device="cuda")
    out.fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.stream(sa):
        # producer: a copy in and an elementwise kernel (x * 1 + 0) per input
        for key in dev:
            tmp = host[key].to("cuda", non_blocking=True)
            torch.add(tmp * 1, 0, out=dev[key])
            tmp.record_stream(sa)
        produced = torch.cuda.Event()
        produced.record(sa)
    with torch.cuda.stream(sb):
        sb.wait_event(produced)
        if path == "two-call":
            rp.relpos_build(dev["q"], dev["rel_pos_h"], dev["rel_pos_w"], H, W, rel_h=rel_h, rel_w=rel_w)
            rp.relpos_attn_fwd(dev["q"], dev["k"], dev["v"], rel_h, rel_w, H, W, d["scale"], out=out)
        else:
            rp.relpos_attn_fused(dev["q"], dev["k"], dev["v"], dev["rel_pos_h"], dev["rel_pos_w"], H, W,
                                 d["scale"], out=out, workspace=ws)
        done = torch.cuda.Event()
        done.record(sb)
    with torch.cuda.stream(sc):
        sc.wait_event(done)
        consumed = out * 1.0
        finished = torch.cuda.Event()
        finished.record(sc)
    finished.synchronize()
    _vs_oracle(f"stream ordering, {path}", consumed, d)
