"""Seeded input generator: determinism, shapes, dtypes and spreads of each workload."""

import pytest
import torch

from relative_position_bias_relpos_amd import inputs


@pytest.mark.parametrize("name", ["tiny", "batched_fp16"])
def test_deterministic(name):
    w = inputs.workload(name, B=1, heads=1) if name != "tiny" else inputs.workload(name)
    a = inputs.make(w, seed=0)
    b = inputs.make(w, seed=0)
    c = inputs.make(w, seed=1)
    for key in ("q", "k", "v", "rel_pos_h", "rel_pos_w"):
        assert torch.equal(a[key], b[key])
        assert not torch.equal(a[key], c[key])


def test_shapes_and_dtypes():
    for name, w in inputs.WORKLOADS.items():
        small = inputs.workload(name, B=1, heads=1)
        d = inputs.make(small)
        assert d["q"].shape == (1, 1, w.H * w.W, 64)
        assert d["rel_pos_h"].shape == (2 * w.H - 1, 64)
        assert d["rel_pos_w"].shape == (2 * w.W - 1, 64)
        assert d["q"].dtype == w.torch_dtype
        assert d["scale"] == 0.125


def test_distributions():
    d = inputs.make(inputs.workload("batched_fp16", B=1, heads=2))
    q = d["q"].float()
    v = d["v"].float()
    assert 3.8 < q.std().item() < 4.2
    assert v.abs().max().item() <= 1.0 and v.min().item() < -0.9
    assert 0.09 < d["rel_pos_h"].float().std().item() < 0.11
    t = inputs.make(inputs.workload("deepencoder", B=1, heads=2))
    assert 0.018 < t["rel_pos_w"].float().std().item() < 0.022


def test_flops_count():
    w = inputs.WORKLOADS["deepencoder"]
    assert w.flops == 4 * 12 * 4096 * 4096 * 64
