"""relpos_attn_fused_noalloc: the fused call on the library's fixed per-device
scratch array instead of a caller workspace.

It runs the same kernels with the same launch as relpos_attn_fused, so its
outputs must equal relpos_attn_fused's bit for bit.  Two no-alloc calls run
back to back, the second on a smaller, ragged problem (the scratch then holds
the first call's leftovers), and the small one is also held to the oracle's
bar (max |gpu - oracle| <= 2e-3, mean <= 1e-4).  A problem whose workspace
exceeds the array is refused before anything is launched.
"""

import numpy as np
import pytest
import torch

from relative_position_bias_relpos_amd import binding as rp
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 96 << 20  # RELPOS_SCRATCH_BYTES in include/relpos.h


def _args(d):
    g = G.to_dev(d)
    return g, (g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], d["H"], d["W"], d["scale"])


def _with_workspace(d, args, out_dtype):
    need = rp.fused_workspace_bytes(*args[0].shape[:2], d["H"], d["W"], args[0].dtype, G.cu_count())
    assert 0 < need <= SCRATCH_BYTES
    ws = torch.full((need,), 0x7f, dtype=torch.uint8, device="cuda")
    out = rp.relpos_attn_fused(*args, out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("out_dtype", [torch.float32, None])
def test_two_calls_large_then_small(out_dtype):
    big = G.make("deepencoder")  # 1 x 12 heads, 64x64, bf16
    small = G.make("rect", B=1, heads=3, H=21, W=35)  # ragged grid, partial units
    print(f"[no-alloc] out_dtype={out_dtype}: 64x64 x 12 then 21x35 x 3", flush=True)
    gb, args_b = _args(big)
    gs, args_s = _args(small)
    odt_b = out_dtype or gb["q"].dtype
    odt_s = out_dtype or gs["q"].dtype
    ref_b = _with_workspace(big, args_b, odt_b)
    ref_s = _with_workspace(small, args_s, odt_s)

    out_b = torch.full(gb["q"].shape, float("nan"), dtype=odt_b, device="cuda")
    out_s = torch.full(gs["q"].shape, float("nan"), dtype=odt_s, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    rp.relpos_attn_fused_noalloc(*args_b, out=out_b)
    rp.relpos_attn_fused_noalloc(*args_s, out=out_s)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before

    assert torch.equal(out_b, ref_b), "64x64: no-alloc call differs from relpos_attn_fused"
    assert torch.equal(out_s, ref_s), "21x35: no-alloc call differs from relpos_attn_fused"
    ref, _, _ = G.oracle_full(small)
    err = np.abs(G.f64(out_s) - ref)
    print(f"[no-alloc] 21x35 vs oracle: max={err.max():.3e} mean={err.mean():.3e}", flush=True)
    assert np.isfinite(err).all()
    if out_dtype is torch.float32:
        assert err.max() <= G.MAX_ABS and err.mean() <= G.MEAN_ABS


def test_too_large_is_refused():
    # 128x128: roundup(H, 4) + roundup(W, 16) = 256 needs more than the array
    # on 256 compute units; on fewer CUs pick a grid that still does not fit.
    H = W = 128
    while rp.fused_workspace_bytes(1, 1, H, W, torch.bfloat16, G.cu_count()) <= SCRATCH_BYTES:
        H += 64
        W += 64
    d = G.make("deepencoder", B=1, heads=1, H=H, W=W)
    g, args = _args(d)
    out = torch.empty(g["q"].shape, dtype=torch.float32, device="cuda")
    with pytest.raises(rp.RelposError) as e:
        rp.relpos_attn_fused_noalloc(*args, out=out)
    assert e.value.status == 2  # E_SHAPE
