"""Windowed blocks: 25 windows of 14x14 (a 64x64 grid padded to 70x70), 12
heads, each window an independent grid with its own 27-row tables.  Every
output of every window against the float64 oracle, through the two-call path
and the fused call, in the launch configurations they choose at this size."""

import numpy as np
import pytest
import torch

from relative_position_bias_relpos_amd import binding as rp
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _check(tag, err):
    print(f"[windowed] {tag}: n={err.size} max={err.max():.3e} mean={err.mean():.3e}", flush=True)
    assert np.isfinite(err).all(), tag
    assert err.max() <= G.MAX_ABS, tag
    assert err.mean() <= G.MEAN_ABS, tag


@pytest.fixture(scope="module")
def case():
    d = G.make("windowed")
    ref, _, _ = G.oracle_full(d)
    return d, ref


def test_two_call_path(case):
    d, ref = case
    out, _, _ = G.gpu_run(d)
    _check("build + attn_fwd", np.abs(G.f64(out) - ref))


def test_two_call_path_with_workspace(case):
    d, ref = case
    g = G.to_dev(d)
    rel_h, rel_w = rp.relpos_build(g["q"], g["rel_pos_h"], g["rel_pos_w"], d["H"], d["W"])
    B, nh = g["q"].shape[:2]
    n = max(rp.workspace_bytes(B, nh, d["H"], d["W"], g["q"].dtype, G.cu_count()), 16)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = rp.relpos_attn_fwd(g["q"], g["k"], g["v"], rel_h, rel_w, d["H"], d["W"], d["scale"], workspace=ws)
    torch.cuda.synchronize()
    _check("build + attn_fwd_ws", np.abs(G.f64(out) - ref))


def test_fused(case):
    d, ref = case
    g = G.to_dev(d)
    out = rp.relpos_attn_fused(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], d["H"], d["W"], d["scale"])
    torch.cuda.synchronize()
    _check("fused", np.abs(G.f64(out) - ref))
