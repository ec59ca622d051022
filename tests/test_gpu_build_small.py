"""relpos_build on small grids (H, W <= 32: the kernel that forms the whole
table products of 32 consecutive queries and writes their rows as one run)
against the float64 oracle's rel_h / rel_w, every (b, h), within the fp32
dot-product bound.

Covers single-row and single-column grids, grids of fewer than 32 queries,
ragged last blocks, runs that start off 16-byte alignment (odd H*W*H), the
largest small grid (32 x 32) and both input dtypes; plus the windowed
workload's shape with many (b, h).
"""

import numpy as np
import pytest
import torch

from oracle import relpos_oracle as O
from relative_position_bias_relpos_amd import binding as rp
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (1, 7), (5, 3), (7, 9), (14, 14), (16, 16), (31, 5), (3, 31), (32, 32), (2, 17), (32, 1)]


def _check_all(d):
    g = G.to_dev(d)
    H, W = d["H"], d["W"]
    rel_h, rel_w = rp.relpos_build(g["q"], g["rel_pos_h"], g["rel_pos_w"], H, W)
    torch.cuda.synchronize()
    B, nh = d["q"].shape[:2]
    worst = 0.0
    for b in range(B):
        for h in range(nh):
            rh, rw = O.rel_tables(G.f64(d["q"][b, h]), G.f64(d["rel_pos_h"]), G.f64(d["rel_pos_w"]), H, W)
            bh, bw = G.build_bound(d, b, h)
            eh = np.abs(G.f64(rel_h[b, h]) - rh)
            ew = np.abs(G.f64(rel_w[b, h]) - rw)
            assert np.isfinite(eh).all() and np.isfinite(ew).all(), (H, W, b, h)
            assert (eh <= bh + 1e-30).all(), (H, W, b, h, float(eh.max()))
            assert (ew <= bw + 1e-30).all(), (H, W, b, h, float(ew.max()))
            worst = max(worst, float(eh.max()), float(ew.max()))
    print(f"[build-small] {H}x{W} {d['q'].dtype} B={B} heads={nh}: max err {worst:.3e}", flush=True)


@pytest.mark.parametrize("H,W", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_small_build(H, W, dtype):
    _check_all(G.make("tiny", seed=H * 37 + W, B=2, heads=3, H=H, W=W, dtype=dtype))


def test_windowed_shape_many_heads():
    _check_all(G.make("windowed", B=5, heads=12))
