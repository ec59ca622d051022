"""Seeded synthetic inputs for relative-position attention workloads.

This module holds no arithmetic of the method: it only draws random numbers and
rounds them to the storage dtype.  Both the HIP path (through the tests and the
benchmark) and the float64 oracle consume the tensors it returns, so the two sides
always see identical rounded values.

Recipe (fixed draw order, so a seed names one input set):
``torch.Generator('cpu').manual_seed(seed)``, then draw, in float32 and in this
order, q, k, v (shape ``[B, heads, H*W, D]``) and the two tables rel_pos_h
``[2H-1, D]`` and rel_pos_w ``[2W-1, D]``; scale each draw, then round to the
workload dtype (round-to-nearest-even, torch ``.to``).

The workloads stand in for DeepEncoder's global attention (the PR #55629 page's
64x64 case), variants of it and its windowed blocks cut into 14x14 windows;
trained tables and real activations are not available, so normal/uniform draws
of the stated spread replace them.
"""

from dataclasses import dataclass, replace

import torch

__all__ = ["Workload", "WORKLOADS", "TAIL_SHAPES", "make", "workload"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    heads: int
    H: int
    W: int
    D: int = 64
    dtype: str = "bf16"          # "bf16" or "fp16"
    qk_mul: float = 1.0          # q, k ~ qk_mul * N(0, 1)
    v_dist: str = "normal"       # "normal": N(0,1); "uniform": U(-1, 1)
    table_std: float = 0.02      # tables ~ N(0, table_std^2)
    scale: float = 0.125
    build_in_step: bool = False  # rel tables built inside the timed call

    @property
    def N(self):
        return self.H * self.W

    @property
    def flops(self):
        """4*B*heads*N^2*D: the two contractions of attention."""
        return 4 * self.B * self.heads * self.N * self.N * self.D

    @property
    def torch_dtype(self):
        return {"bf16": torch.bfloat16, "fp16": torch.float16}[self.dtype]


WORKLOADS = {
    "tiny": Workload("tiny", B=1, heads=2, H=16, W=16),
    "deepencoder": Workload("deepencoder", B=1, heads=12, H=64, W=64),
    "batched_fp16": Workload("batched_fp16", B=4, heads=12, H=64, W=64, dtype="fp16",
                             qk_mul=4.0, v_dist="uniform", table_std=0.1),
    "rect": Workload("rect", B=2, heads=12, H=48, W=80),
    "vitl": Workload("vitl", B=2, heads=16, H=96, W=96, build_in_step=True),
    # Windowed blocks: the 64x64 grid padded to 70x70 and cut into 25 windows of
    # 14x14, each an independent grid with its own 27-row tables; B counts the
    # windows of one image.  The window size is not on the PR #55629 page (its
    # windowed blocks stay on SDPA); 14 is a stand-in.
    "windowed": Workload("windowed", B=25, heads=12, H=14, W=14),
}

# Grids whose token count is not a multiple of any tile size: correctness only.
TAIL_SHAPES = [(14, 14), (7, 9), (1, 1), (1, 37), (37, 1), (40, 40), (63, 65), (5, 3), (2, 17)]


def workload(name, **overrides):
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def make(w, seed=0):
    """Draw one input set for workload ``w``; returns a dict of CPU tensors."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    shape = (w.B, w.heads, w.N, w.D)
    q = torch.randn(shape, generator=g, dtype=torch.float32) * w.qk_mul
    k = torch.randn(shape, generator=g, dtype=torch.float32) * w.qk_mul
    if w.v_dist == "normal":
        v = torch.randn(shape, generator=g, dtype=torch.float32)
    elif w.v_dist == "uniform":
        v = torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    else:
        raise ValueError(w.v_dist)
    th = torch.randn((2 * w.H - 1, w.D), generator=g, dtype=torch.float32) * w.table_std
    tw = torch.randn((2 * w.W - 1, w.D), generator=g, dtype=torch.float32) * w.table_std
    dt = w.torch_dtype
    return {
        "q": q.to(dt), "k": k.to(dt), "v": v.to(dt),
        "rel_pos_h": th.to(dt), "rel_pos_w": tw.to(dt),
        "H": w.H, "W": w.W, "scale": w.scale,
    }
