"""Degenerate and extreme scalars against the float64 oracle.

* scale = 0 (the scores are the bias alone) and a negative scale, on ragged
  grids (masked key cells) and a tile-aligned one, through every launch
  configuration and the fused call.
* bf16 v of large magnitude (|v| up to 60000, inside the documented fp16
  staging range), compared in units of the draw's spread.
"""

import numpy as np
import pytest
import torch

from relative_position_bias_relpos_amd import binding as rp
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _check(tag, err, unit=1.0):
    err = err / unit
    print(f"[scale-range] {tag}: n={err.size} max={err.max():.3e} mean={err.mean():.3e}", flush=True)
    assert np.isfinite(err).all(), tag
    assert err.max() <= G.MAX_ABS, tag
    assert err.mean() <= G.MEAN_ABS, tag


SHAPES = [("tiny", dict(B=1, heads=3, H=7, W=9)), ("rect", dict(B=1, heads=3, H=21, W=35)),
          ("tiny", dict(B=1, heads=2, H=16, W=32))]


@pytest.mark.parametrize("scale", [0.0, -0.125])
@pytest.mark.parametrize("cfg", [0, 1, 3, 5])
@pytest.mark.parametrize("name,kw", SHAPES)
def test_scale_two_call_path(scale, cfg, name, kw):
    d = G.make(name, **kw)
    d["scale"] = scale
    out, _, _ = G.gpu_run(d, config=cfg)
    ref, _, _ = G.oracle_full(d)
    _check(f"scale={scale} cfg{cfg} {kw['H']}x{kw['W']}", np.abs(G.f64(out) - ref))


@pytest.mark.parametrize("scale", [0.0, -0.125])
@pytest.mark.parametrize("name,kw", SHAPES)
def test_scale_fused(scale, name, kw):
    d = G.make(name, **kw)
    d["scale"] = scale
    g = G.to_dev(d)
    out = rp.relpos_attn_fused(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], d["H"], d["W"], scale)
    torch.cuda.synchronize()
    ref, _, _ = G.oracle_full(d)
    _check(f"fused scale={scale} {kw['H']}x{kw['W']}", np.abs(G.f64(out) - ref))


def test_scale_zero_full_size_sampled():
    """scale = 0 on the 64x64 workload in its default launch."""
    d = G.make("deepencoder", B=1, heads=2)
    d["scale"] = 0.0
    out, _, _ = G.gpu_run(d)
    _check("scale=0 64x64 sampled", G.oracle_sampled(d, out, 96))


def test_tiny_nonzero_scale_rejected():
    d = G.make("tiny")
    g = G.to_dev(d)
    rel_h, rel_w = rp.relpos_build(g["q"], g["rel_pos_h"], g["rel_pos_w"], d["H"], d["W"])
    with pytest.raises(rp.RelposError) as e:
        rp.relpos_attn_fwd(g["q"], g["k"], g["v"], rel_h, rel_w, d["H"], d["W"], 2.0 ** -70)
    assert e.value.status == 9  # E_VALUE


@pytest.mark.parametrize("cfg", [None, 1, 3, 5])
def test_large_bf16_v(cfg):
    """v ~ 16384 * N(0, 1), clipped to +-60000, in bf16: staged as fp16 without
    overflow.  Errors are measured in units of 16384."""
    d = G.make("rect", B=1, heads=2, H=24, W=40)
    g = torch.Generator().manual_seed(11)
    v = (torch.randn(d["v"].shape, generator=g) * 16384.0).clamp_(-60000.0, 60000.0)
    d["v"] = v.to(torch.bfloat16)
    out, _, _ = G.gpu_run(d, config=cfg)
    ref, _, _ = G.oracle_full(d)
    _check(f"large bf16 v cfg{cfg}", np.abs(G.f64(out) - ref), unit=16384.0)
    gx = G.to_dev(d)
    fused = rp.relpos_attn_fused(gx["q"], gx["k"], gx["v"], gx["rel_pos_h"], gx["rel_pos_w"], d["H"], d["W"],
                                 d["scale"])
    torch.cuda.synchronize()
    _check("large bf16 v fused", np.abs(G.f64(fused) - ref), unit=16384.0)
