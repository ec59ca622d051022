"""Parity of the HIP path (through the C ABI) against the float64 oracle.

Bar: max |gpu - oracle| <= 2e-3 and mean <= 1e-4 on the attention output (fp32
out); rel_h/rel_w within the fp32 dot-product forward-error bound.  Small and
ragged grids are compared element by element over every output, in every
launch configuration; the full-size workloads are compared over every output
in tests/test_gpu_full_parity.py.
"""

import gc

import numpy as np
import pytest
import torch

from relative_position_bias_relpos_amd import inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _report(tag, err):
    print(f"[parity] {tag}: n={err.size} max={err.max():.3e} mean={err.mean():.3e}", flush=True)


def _check(tag, err):
    _report(tag, err)
    assert np.isfinite(err).all(), tag
    assert err.max() <= G.MAX_ABS, tag
    assert err.mean() <= G.MEAN_ABS, tag


# ---- relpos_build -----------------------------------------------------------

@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_build_within_fp32_dot_bound(name):
    d = G.make(name)
    print(f"[build] {name}", flush=True)
    _, rel_h, rel_w = G.gpu_run(d)
    from oracle import relpos_oracle as O
    B, nh = d["q"].shape[:2]
    pairs = [(b, h) for b in range(B) for h in range(nh)][:4]
    for b, h in pairs:
        rh, rw = O.rel_tables(G.f64(d["q"][b, h]), G.f64(d["rel_pos_h"]), G.f64(d["rel_pos_w"]), d["H"], d["W"])
        bh, bw = G.build_bound(d, b, h)
        eh = np.abs(G.f64(rel_h[b, h]) - rh)
        ew = np.abs(G.f64(rel_w[b, h]) - rw)
        assert (eh <= bh + 1e-30).all(), (name, b, h, float(eh.max()))
        assert (ew <= bw + 1e-30).all(), (name, b, h, float(ew.max()))


# ---- attention, every output -------------------------------------------------

def test_tiny_full():
    d = G.make("tiny")
    out, _, _ = G.gpu_run(d)
    ref, _, _ = G.oracle_full(d)
    _check("tiny", np.abs(G.f64(out) - ref))


@pytest.mark.parametrize("H,W", inputs.TAIL_SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_tail_shapes_full(H, W, dtype):
    d = G.make("tiny", seed=H * 100 + W, H=H, W=W, dtype=dtype)
    print(f"[tail] {H}x{W} {dtype}", flush=True)
    out, _, _ = G.gpu_run(d)
    ref, _, _ = G.oracle_full(d)
    _check(f"tail {H}x{W} {dtype}", np.abs(G.f64(out) - ref))


def test_small_stress_fp16_full():
    """fp16, q,k ~ 4 N(0,1), tables ~ N(0, 0.1^2): large logits on a small grid."""
    d = G.make("batched_fp16", B=1, heads=3, H=12, W=20)
    out, _, _ = G.gpu_run(d)
    ref, _, _ = G.oracle_full(d)
    _check("stress fp16 12x20", np.abs(G.f64(out) - ref))


# ---- properties on the GPU ---------------------------------------------------

def test_ones_v_gives_ones():
    d = G.make("rect", B=1, heads=2, H=24, W=40)
    d["v"] = torch.ones_like(d["v"])
    out, _, _ = G.gpu_run(d)
    assert (out - 1.0).abs().max().item() <= 1e-5


def test_per_query_constant_in_rel_h_is_invisible():
    d = G.make("deepencoder", B=1, heads=2)
    g = G.to_dev(d)
    from relative_position_bias_relpos_amd import binding as rp
    rel_h, rel_w = rp.relpos_build(g["q"], g["rel_pos_h"], g["rel_pos_w"], d["H"], d["W"])
    base = rp.relpos_attn_fwd(g["q"], g["k"], g["v"], rel_h, rel_w, d["H"], d["W"], d["scale"])
    c = torch.randn(rel_h.shape[:-1] + (1,), device="cuda", generator=torch.Generator("cuda").manual_seed(3)) * 4
    sh = rp.relpos_attn_fwd(g["q"], g["k"], g["v"], rel_h + c, rel_w - 0.5 * c, d["H"], d["W"], d["scale"])
    torch.cuda.synchronize()
    assert (sh - base).abs().max().item() <= G.MAX_ABS


def test_half_precision_output():
    for dtype in ("bf16", "fp16"):
        d = G.make("tiny", dtype=dtype)
        out, _, _ = G.gpu_run(d, out_dtype=d["q"].dtype)
        assert out.dtype == d["q"].dtype
        ref, _, _ = G.oracle_full(d)
        err = np.abs(G.f64(out) - ref)
        ulp = 2.0 ** (-8 if dtype == "bf16" else -11)
        assert (err <= G.MAX_ABS + ulp * np.abs(ref)).all(), dtype
        print(f"[parity] tiny out={dtype}: max={err.max():.3e} mean={err.mean():.3e}", flush=True)


def test_run_to_run_bitwise():
    d = G.make("rect", B=1, heads=3)
    a, ha, wa = G.gpu_run(d)
    b, hb, wb = G.gpu_run(d)
    assert torch.equal(a, b) and torch.equal(ha, hb) and torch.equal(wa, wb)


def test_no_allocation_during_calls():
    d = G.make("deepencoder")
    g = G.to_dev(d)
    from relative_position_bias_relpos_amd import binding as rp
    H, W = d["H"], d["W"]
    rel_h = torch.empty(g["q"].shape[:3] + (H,), dtype=torch.float32, device="cuda")
    rel_w = torch.empty(g["q"].shape[:3] + (W,), dtype=torch.float32, device="cuda")
    out = torch.empty(g["q"].shape, dtype=torch.float32, device="cuda")
    rp.relpos_build(g["q"], g["rel_pos_h"], g["rel_pos_w"], H, W, rel_h=rel_h, rel_w=rel_w)
    rp.relpos_attn_fwd(g["q"], g["k"], g["v"], rel_h, rel_w, H, W, d["scale"], out=out)
    torch.cuda.synchronize()
    gc.collect()  # tensors of earlier tests must not be freed inside the measured loop
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    free_before, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        rp.relpos_build(g["q"], g["rel_pos_h"], g["rel_pos_w"], H, W, rel_h=rel_h, rel_w=rel_w)
        rp.relpos_attn_fwd(g["q"], g["k"], g["v"], rel_h, rel_w, H, W, d["scale"], out=out)
    torch.cuda.synchronize()
    free_after, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() <= before
    assert torch.cuda.max_memory_allocated() == before  # the peak never rose above the start
    # A dense bf16 bias for this workload would be 384 MiB; nothing of that order appears.
    assert abs(free_before - free_after) < 2 * 1024 * 1024


# ---- every launch configuration ------------------------------------------------

@pytest.mark.parametrize("cfg", [0, 1, 3, 5, 6])
@pytest.mark.parametrize("name,kw", [("tiny", {}), ("rect", dict(B=1, heads=2, H=21, W=35)),
                                     ("batched_fp16", dict(B=1, heads=2, H=20, W=24))])
def test_each_launch_config(cfg, name, kw):
    d = G.make(name, **kw)
    out, _, _ = G.gpu_run(d, config=cfg)
    ref, _, _ = G.oracle_full(d)
    _check(f"cfg{cfg} {name}", np.abs(G.f64(out) - ref))


@pytest.mark.parametrize("name", ["deepencoder", "rect", "batched_fp16", "windowed"])
def test_automatic_config_matches_its_prediction(name):
    """relpos_attn_fwd launches the configuration relpos_attn_config predicts
    for this device: the same bits as forcing it through relpos_attn_fwd_cfg."""
    from relative_position_bias_relpos_amd import binding as rp
    d = G.make(name)
    auto, _, _ = G.gpu_run(d)
    B, nh = d["q"].shape[:2]
    cfg = rp.attn_config(B, nh, d["H"], d["W"], d["q"].dtype, G.cu_count())
    forced, _, _ = G.gpu_run(d, config=cfg)
    assert torch.equal(auto, forced), (name, cfg)


# ---- key-range split (relpos_attn_fwd_ws) ----------------------------------------

def _run_split(d, ws, config=None):
    from relative_position_bias_relpos_amd import binding as rp
    g = G.to_dev(d)
    rel_h, rel_w = rp.relpos_build(g["q"], g["rel_pos_h"], g["rel_pos_w"], d["H"], d["W"])
    out = rp.relpos_attn_fwd(g["q"], g["k"], g["v"], rel_h, rel_w, d["H"], d["W"], d["scale"], workspace=ws,
                             config=config)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("tiny", dict(H=14, W=14)), ("tiny", dict(H=7, W=9, dtype="fp16")),
                                     ("rect", dict(B=1, heads=3, H=21, W=35)),
                                     ("batched_fp16", dict(B=1, heads=2, H=20, W=24))])
def test_forced_split_full(name, kw):
    """Forced split on small grids: every unit is in the last round, cut into a
    head and a tail (down to one tile each) that are merged afterwards."""
    d = G.make(name, **kw)
    ws = torch.full((G.split_ws_bytes(),), 0x7f, dtype=torch.uint8, device="cuda")  # contents are not read
    out = _run_split(d, ws, config=5)
    ref, _, _ = G.oracle_full(d)
    _check(f"split {name} {kw}", np.abs(G.f64(out) - ref))
    again = _run_split(d, ws, config=5)
    assert torch.equal(out, again), "split result depends on arrival order"


def test_split_chosen_with_a_workspace():
    """relpos_attn_fwd_ws with a workspace splits 16 fp16 heads of 96x96 (the
    cost model's choice there) and asks for the documented workspace size."""
    from relative_position_bias_relpos_amd import binding as rp
    d = G.make("vitl", B=1, dtype="fp16")
    B, nh = d["q"].shape[:2]
    assert rp.attn_config(B, nh, d["H"], d["W"], d["q"].dtype, G.cu_count(), with_workspace=True) == 5
    assert rp.workspace_bytes(B, nh, d["H"], d["W"], d["q"].dtype, G.cu_count()) == G.split_ws_bytes()
    ws = torch.empty(G.split_ws_bytes(), dtype=torch.uint8, device="cuda")
    out = _run_split(d, ws)
    assert torch.equal(out, _run_split(d, ws, config=5))


def test_split_workspace_errors():
    from relative_position_bias_relpos_amd import binding as rp
    d = G.make("vitl", B=1, dtype="fp16")  # 16 fp16 heads of 96x96: the cost model splits it
    g = G.to_dev(d)
    rel_h, rel_w = rp.relpos_build(g["q"], g["rel_pos_h"], g["rel_pos_w"], d["H"], d["W"])
    small = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(rp.RelposError) as e:
        rp.relpos_attn_fwd(g["q"], g["k"], g["v"], rel_h, rel_w, d["H"], d["W"], d["scale"], workspace=small)
    assert e.value.status == 2  # E_SHAPE: workspace too small
    big = torch.zeros(G.split_ws_bytes() + g["q"].numel() * 4, dtype=torch.uint8, device="cuda")
    out = big[: g["q"].numel() * 4].view(torch.float32).view(g["q"].shape)
    with pytest.raises(rp.RelposError) as e:
        rp.relpos_attn_fwd(g["q"], g["k"], g["v"], rel_h, rel_w, d["H"], d["W"], d["scale"], out=out, workspace=big)
    assert e.value.status == 6  # E_ALIAS: the workspace overlaps out
    with pytest.raises(rp.RelposError) as e:
        rp.relpos_attn_fwd(g["q"], g["k"], g["v"], rel_h, rel_w, d["H"], d["W"], d["scale"], config=5)
    assert e.value.status == 1  # E_NULL: the forced split without a workspace


def test_split_workspace_reused_across_shapes():
    """One workspace for split problems of different shapes in turn."""
    ws = torch.empty(G.split_ws_bytes(), dtype=torch.uint8, device="cuda")
    for d in (G.make("deepencoder", B=1, heads=2), G.make("rect", B=1, heads=6), G.make("deepencoder", B=1, heads=2)):
        out = _run_split(d, ws, config=5)
        unsplit = _run_split(d, None)
        assert (out - unsplit).abs().max().item() <= G.MAX_ABS
        assert torch.equal(out, _run_split(d, ws, config=5))


@pytest.mark.parametrize("cfg", [0, 5])
@pytest.mark.parametrize("H,W", [(12, 32), (72, 16), (76, 16)])
def test_rel_h_rows_in_lds_shapes(cfg, H, W):
    """8-wave launches copy each unit's rel_h rows to LDS on tile-aligned grids
    with H <= 72: a last unit whose upper waves lie past the grid (12x32: 384
    queries), the largest H of that path (72: nine 16-byte chunks per lane, and
    a half-empty last unit) and the first H past it (76: rel_h read from memory)."""
    d = G.make("tiny", H=H, W=W)
    ws = torch.empty(G.split_ws_bytes(), dtype=torch.uint8, device="cuda") if cfg == 5 else None
    out = _run_split(d, ws, config=cfg)
    ref, _, _ = G.oracle_full(d)
    _check(f"cfg{cfg} rel_h rows {H}x{W}", np.abs(G.f64(out) - ref))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_forced_split_half_precision_output(dtype):
    """The merge kernel's bf16/fp16 stores, against the oracle."""
    d = G.make("tiny", dtype=dtype, H=14, W=18)
    out, _, _ = G.gpu_run(d, out_dtype=d["q"].dtype, config=5)
    assert out.dtype == d["q"].dtype
    ref, _, _ = G.oracle_full(d)
    err = np.abs(G.f64(out) - ref)
    ulp = 2.0 ** (-8 if dtype == "bf16" else -11)
    assert (err <= G.MAX_ABS + ulp * np.abs(ref)).all(), dtype
    print(f"[parity] split tiny 14x18 out={dtype}: max={err.max():.3e} mean={err.mean():.3e}", flush=True)
