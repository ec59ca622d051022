"""Launch configuration 6 (the 12-wave kernel: 6 query blocks x even/odd key
tiles per workgroup, merged in LDS) against the float64 oracle, every output.

Covers tile-aligned and ragged grids, workgroups spanning two heads (the block
count per head is not a multiple of 6), a last workgroup with blocks past the
end, an odd number of key tiles (the odd waves' last step idle), both input
dtypes, half-precision outputs, scale 0 and a negative scale, and large bf16 v.
"""

import numpy as np
import pytest
import torch

from relative_position_bias_relpos_amd import binding as rp
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

CFG = 6


def _check(tag, err, unit=1.0):
    err = err / unit
    print(f"[attn12] {tag}: n={err.size} max={err.max():.3e} mean={err.mean():.3e}", flush=True)
    assert np.isfinite(err).all(), tag
    assert err.max() <= G.MAX_ABS, tag
    assert err.mean() <= G.MEAN_ABS, tag


SHAPES = [
    ("tiny", dict(B=1, heads=2, H=16, W=16)),      # 8 blocks per head: workgroups span two heads
    ("tiny", dict(B=1, heads=3, H=16, W=32)),      # aligned, 16 blocks per head
    ("tiny", dict(B=2, heads=3, H=14, W=14)),      # ragged both ways, 7 blocks per head
    ("rect", dict(B=1, heads=3, H=21, W=35)),      # ragged, odd tile count (6 x 3 = 18? see below)
    ("tiny", dict(B=1, heads=2, H=5, W=48)),       # ragged rows: 2 x 3 = 6 tiles
    ("tiny", dict(B=1, heads=2, H=4, W=80)),       # one tile row: 5 tiles (odd), band_tiles = 1
    ("tiny", dict(B=1, heads=1, H=1, W=200)),      # a single grid row, 13 tiles
    ("tiny", dict(B=1, heads=5, H=63, W=65)),      # large ragged grid
    ("batched_fp16", dict(B=1, heads=3, H=20, W=24)),
    ("batched_fp16", dict(B=2, heads=2, H=40, W=40)),
]


@pytest.mark.parametrize("name,kw", SHAPES)
def test_parity(name, kw):
    d = G.make(name, **kw)
    print(f"[attn12] {name} {kw}", flush=True)
    out, _, _ = G.gpu_run(d, config=CFG)
    ref, _, _ = G.oracle_full(d)
    _check(f"{name} {kw}", np.abs(G.f64(out) - ref))
    again, _, _ = G.gpu_run(d, config=CFG)
    assert torch.equal(out, again), "not reproducible run to run"


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_half_precision_output(dtype):
    d = G.make("tiny", dtype=dtype, B=1, heads=3, H=14, W=18)
    out, _, _ = G.gpu_run(d, out_dtype=d["q"].dtype, config=CFG)
    assert out.dtype == d["q"].dtype
    ref, _, _ = G.oracle_full(d)
    err = np.abs(G.f64(out) - ref)
    ulp = 2.0 ** (-8 if dtype == "bf16" else -11)
    assert (err <= G.MAX_ABS + ulp * np.abs(ref)).all(), dtype
    print(f"[attn12] out={dtype}: max={err.max():.3e} mean={err.mean():.3e}", flush=True)


@pytest.mark.parametrize("scale", [0.0, -0.125])
@pytest.mark.parametrize("kw", [dict(B=1, heads=3, H=21, W=35), dict(B=1, heads=2, H=16, W=32)])
def test_scale(scale, kw):
    d = G.make("rect", **kw)
    d["scale"] = scale
    out, _, _ = G.gpu_run(d, config=CFG)
    ref, _, _ = G.oracle_full(d)
    _check(f"scale={scale} {kw}", np.abs(G.f64(out) - ref))


def test_large_bf16_v():
    d = G.make("rect", B=1, heads=2, H=24, W=40)
    g = torch.Generator().manual_seed(11)
    v = (torch.randn(d["v"].shape, generator=g) * 16384.0).clamp_(-60000.0, 60000.0)
    d["v"] = v.to(torch.bfloat16)
    out, _, _ = G.gpu_run(d, config=CFG)
    ref, _, _ = G.oracle_full(d)
    _check("large bf16 v", np.abs(G.f64(out) - ref), unit=16384.0)


def test_too_few_blocks_per_head_is_refused():
    """Fewer than 6 query blocks of 32 per head (N <= 160): E_SHAPE."""
    d = G.make("tiny", H=10, W=16)
    with pytest.raises(rp.RelposError) as e:
        G.gpu_run(d, config=CFG)
    assert e.value.status == 2


def test_no_allocation():
    d = G.make("deepencoder", B=1, heads=4)
    g = G.to_dev(d)
    H, W = d["H"], d["W"]
    rel_h, rel_w = rp.relpos_build(g["q"], g["rel_pos_h"], g["rel_pos_w"], H, W)
    out = torch.empty(g["q"].shape, dtype=torch.float32, device="cuda")
    call = lambda: rp.relpos_attn_fwd(g["q"], g["k"], g["v"], rel_h, rel_w, H, W, d["scale"], out=out, config=CFG)
    call()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == before
