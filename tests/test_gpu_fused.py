"""relpos_attn_fused (bias computed inside the attention kernel) against the
float64 oracle and against the two-call path relpos_build + relpos_attn_fwd.

Same bar as the two-call path: max |gpu - oracle| <= 2e-3, mean <= 1e-4 (fp32
out), every output on small and ragged grids, sampled rows at full size.
"""

import ctypes

import gc

import numpy as np
import pytest
import torch

from relative_position_bias_relpos_amd import binding as rp
from relative_position_bias_relpos_amd import inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _check(tag, err):
    print(f"[fused] {tag}: n={err.size} max={err.max():.3e} mean={err.mean():.3e}", flush=True)
    assert np.isfinite(err).all(), tag
    assert err.max() <= G.MAX_ABS, tag
    assert err.mean() <= G.MEAN_ABS, tag


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _small_grid(H, W):
    """Grids whose bias rows the 16-query kernel forms in LDS: H, W <= 32 and
    at most four key tiles of 4 grid rows x 16 columns."""
    return H <= 32 and W <= 32 and ((H + 3) // 4) * ((W + 15) // 16) <= 4


def _ws_bytes(H, W, BH=2, dtype="bf16"):
    """The size include/relpos.h documents for relpos_attn_fused: none on small
    grids, the 12-wave kernel's slots where it runs (bf16, W % 32 == 0,
    H % 4 == 0, N >= 2048: one per b*heads when H, W <= 64, else one per
    workgroup), else the split-grid kernel's pieces and bias slots."""
    if _small_grid(H, W):
        return 0
    if dtype == "bf16" and W % 32 == 0 and H % 4 == 0 and H * W >= 2048:
        units = (BH * ((H * W + 31) // 32) + 5) // 6
        slots = min(units, _cus())
        if H <= 64 and W <= 64:  # slots only for units spanning two heads or partial: one per b*heads
            slots = min(slots, BH)
        return slots * 6 * 32 * (H + W) * 4
    rows = (H + 3) // 4 * 4 + (W + 15) // 16 * 16
    return _cus() * (2 * (256 * 64 + 2 * 256) + 256 * rows) * 4


def _fused(d, ws=None, out_dtype=torch.float32):
    g = G.to_dev(d)
    out = rp.relpos_attn_fused(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], d["H"], d["W"],
                               d["scale"], out_dtype=out_dtype, workspace="auto" if ws is None else ws)
    torch.cuda.synchronize()
    return out


def _filled_ws(H, W, byte):
    # The workspace is scratch: whatever it holds on entry must not matter
    # (0x7f.. is a large finite float, 0xff.. a NaN pattern).
    return torch.full((_ws_bytes(H, W),), byte, dtype=torch.uint8, device="cuda")


def test_workspace_size_matches_header():
    for H, W in ((64, 64), (48, 80), (7, 9), (1, 1), (32, 32), (96, 96), (14, 14), (16, 16), (20, 12), (4, 48)):
        assert rp.fused_workspace_bytes(1, 2, H, W, torch.bfloat16, _cus()) == _ws_bytes(H, W)
        assert rp.fused_workspace_bytes(1, 2, H, W, torch.float16, _cus()) == _ws_bytes(H, W, dtype="fp16")
    assert rp.fused_workspace_bytes(4, 12, 64, 64, torch.bfloat16, _cus()) == _ws_bytes(64, 64, BH=48)


# ---- the 12-wave fused kernel (bf16, W % 32 == 0, H % 4 == 0, N >= 2048) -------------

@pytest.mark.parametrize("name,kw", [
    ("tiny", dict(B=1, heads=1, H=32, W=64)),    # 11 units, the last with 4 of 6 blocks
    ("tiny", dict(B=1, heads=3, H=32, W=64)),    # 64 blocks per head: units span two heads
    ("tiny", dict(B=2, heads=15, H=32, W=64)),   # 320 units: workgroups take two units in turn
    ("rect", dict(B=1, heads=2, H=36, W=96)),    # 36 rows: a column band of 9 tiles
])
def test_twelve_wave_fused_full(name, kw):
    d = G.make(name, **kw)
    assert rp.fused_workspace_bytes(d["q"].shape[0], d["q"].shape[1], d["H"], d["W"], d["q"].dtype, _cus()) == \
        _ws_bytes(d["H"], d["W"], BH=d["q"].shape[0] * d["q"].shape[1])
    print(f"[fused] 12-wave {name} {kw}", flush=True)
    ref, _, _ = G.oracle_full(d)
    out = _fused(d, _filled_ws(d["H"], d["W"], 0x7f) if d["q"].shape[0] * d["q"].shape[1] <= 2 else None)
    _check(f"12-wave {name} {kw}", np.abs(G.f64(out) - ref))
    two, _, _ = G.gpu_run(d)
    assert (out - two).abs().max().item() <= G.MAX_ABS
    assert torch.equal(out, _fused(d)), "run-to-run difference"


@pytest.mark.parametrize("kw", [
    dict(B=1, heads=2, H=64, W=64),   # 43 units: LDS-resident bias, one unit spanning two heads, a partial last unit
    dict(B=1, heads=3, H=48, W=64),   # 48 units, none spanning two heads: all bias rows in LDS
    dict(B=1, heads=2, H=64, W=32),   # rows of 32 columns in the 64-column LDS rows
    dict(B=3, heads=4, H=40, W=64),   # 160 units on fewer workgroups than units when CUs < 160
])
def test_twelve_wave_fused_lds_bias(kw):
    """Grids with H, W <= 64: units inside one head keep their bias rows in
    LDS, the others in the workspace slot; every output against the oracle,
    and bit for bit against the two-call path (same products, same order)."""
    d = G.make("tiny", **kw)
    print(f"[fused] LDS bias {kw}", flush=True)
    ref, _, _ = G.oracle_full(d)
    out = _fused(d)
    _check(f"LDS bias {kw}", np.abs(G.f64(out) - ref))
    two, _, _ = G.gpu_run(d, config=6)  # the same 12-wave kernel in the two-call path
    assert torch.equal(out, two), "fused call differs from relpos_build + relpos_attn_fwd"


def test_twelve_wave_fused_lds_bias_more_heads_than_workgroups():
    """300 heads of 32x64: more b*heads than workgroups, so the units spanning
    two heads use per-workgroup slots; bitwise against the two-call path on
    the same kernel, and every output of three heads against the oracle."""
    d = G.make("tiny", B=25, heads=12, H=32, W=64)
    BH = 300
    assert rp.fused_workspace_bytes(25, 12, 32, 64, torch.bfloat16, _cus()) == _ws_bytes(32, 64, BH=BH)
    out = _fused(d)
    two, _, _ = G.gpu_run(d, config=6)
    assert torch.equal(out, two), "fused call differs from relpos_build + relpos_attn_fwd"
    for b, h in ((0, 0), (12, 5), (24, 11)):  # first, a middle and the last head
        sub = {**d, **{n: d[n][b:b + 1, h:h + 1] for n in ("q", "k", "v")}}
        ref, _, _ = G.oracle_full(sub)
        _check(f"300 heads, head ({b}, {h})", np.abs(G.f64(out[b:b + 1, h:h + 1]) - ref))


@pytest.mark.parametrize("scale", [0.0, -0.125])
@pytest.mark.parametrize("H", [32, 64])
def test_twelve_wave_fused_scale(scale, H):
    d = G.make("tiny", B=1, heads=2, H=H, W=64)
    d["scale"] = scale
    ref, _, _ = G.oracle_full(d)
    _check(f"12-wave scale {scale}", np.abs(G.f64(_fused(d)) - ref))


def test_twelve_wave_fused_half_output():
    d = G.make("tiny", B=1, heads=2, H=32, W=64)
    out = _fused(d, out_dtype=torch.bfloat16)
    ref, _, _ = G.oracle_full(d)
    err = np.abs(G.f64(out) - ref)
    assert (err <= G.MAX_ABS + 2.0 ** -8 * np.abs(ref)).all()


def test_tiny_full():
    d = G.make("tiny")
    ref, _, _ = G.oracle_full(d)
    _check("tiny", np.abs(G.f64(_fused(d, _filled_ws(d["H"], d["W"], 0xff))) - ref))


@pytest.mark.parametrize("H,W", inputs.TAIL_SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_tail_shapes_full(H, W, dtype):
    d = G.make("tiny", seed=H * 100 + W, H=H, W=W, dtype=dtype)
    print(f"[fused] tail {H}x{W} {dtype}", flush=True)
    ref, _, _ = G.oracle_full(d)
    out = _fused(d, _filled_ws(H, W, 0x7f))
    _check(f"tail {H}x{W} {dtype}", np.abs(G.f64(out) - ref))
    assert torch.equal(out, _fused(d, _filled_ws(H, W, 0xff))), "result depends on workspace contents"


@pytest.mark.parametrize("name,kw", [("batched_fp16", dict(B=1, heads=3, H=12, W=20)),
                                     ("rect", dict(B=2, heads=3, H=21, W=35)),
                                     ("tiny", dict(B=3, heads=5, H=9, W=31)),
                                     ("tiny", dict(B=1, heads=2, H=33, W=8))])
def test_small_grids_full(name, kw):
    """Waves whose 32 queries span several grid rows (W < 32), a grid row
    boundary inside a wave (W = 20, 35), and units with queries past the grid."""
    d = G.make(name, **kw)
    ref, _, _ = G.oracle_full(d)
    _check(f"{name} {kw}", np.abs(G.f64(_fused(d)) - ref))


def test_ones_v_gives_ones():
    d = G.make("rect", B=1, heads=2, H=24, W=40)
    d["v"] = torch.ones_like(d["v"])
    assert (_fused(d) - 1.0).abs().max().item() <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_half_precision_output(dtype):
    d = G.make("tiny", dtype=dtype, H=14, W=18)
    out = _fused(d, out_dtype=d["q"].dtype)
    assert out.dtype == d["q"].dtype
    ref, _, _ = G.oracle_full(d)
    err = np.abs(G.f64(out) - ref)
    ulp = 2.0 ** (-8 if dtype == "bf16" else -11)
    assert (err <= G.MAX_ABS + ulp * np.abs(ref)).all(), dtype
    print(f"[fused] tiny 14x18 out={dtype}: max={err.max():.3e} mean={err.mean():.3e}", flush=True)


def test_workspace_reused_across_shapes():
    """One workspace, problems whose bias rows have different strides in turn."""
    ws = torch.empty(max(_ws_bytes(64, 64), _ws_bytes(48, 80), _ws_bytes(7, 9)), dtype=torch.uint8, device="cuda")
    cases = [G.make("deepencoder", B=1, heads=2), G.make("tiny", H=7, W=9), G.make("rect", B=1, heads=4),
             G.make("deepencoder", B=1, heads=2)]
    for d in cases:
        out = _fused(d, ws)
        two, _, _ = G.gpu_run(d)
        assert (out - two).abs().max().item() <= G.MAX_ABS
        assert torch.equal(out, _fused(d, ws))


def test_workspace_errors():
    d = G.make("deepencoder", B=1, heads=2)
    g = G.to_dev(d)
    H, W = d["H"], d["W"]
    small = torch.zeros(_ws_bytes(H, W) - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(rp.RelposError) as e:
        rp.relpos_attn_fused(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], H, W, d["scale"],
                             workspace=small)
    assert e.value.status == 2  # E_SHAPE: workspace too small
    big = torch.zeros(_ws_bytes(H, W) + g["q"].numel() * 4, dtype=torch.uint8, device="cuda")
    out = big[: g["q"].numel() * 4].view(torch.float32).view(g["q"].shape)
    with pytest.raises(rp.RelposError) as e:
        rp.relpos_attn_fused(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], H, W, d["scale"],
                             out=out, workspace=big)
    assert e.value.status == 6  # E_ALIAS: the workspace overlaps out
    lib = rp._load()
    st = lib.relpos_attn_fused(rp._ptr(g["q"]), rp._ptr(g["k"]), rp._ptr(g["v"]), rp._ptr(g["rel_pos_h"]),
                               rp._ptr(g["rel_pos_w"]), rp._ptr(big), 1, 2, H, W, 64, float(d["scale"]),
                               rp.RELPOS_BF16, rp.RELPOS_FP32, ctypes.c_void_p(0), 1 << 30, ctypes.c_void_p(0))
    assert st == 1  # E_NULL: no workspace


def test_no_allocation_during_calls():
    d = G.make("deepencoder")
    g = G.to_dev(d)
    H, W = d["H"], d["W"]
    out = torch.empty(g["q"].shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(_ws_bytes(H, W, BH=12), dtype=torch.uint8, device="cuda")
    call = lambda: rp.relpos_attn_fused(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], H, W,
                                        d["scale"], out=out, workspace=ws)
    call()
    torch.cuda.synchronize()
    gc.collect()  # tensors of earlier tests must not be freed inside the measured loop
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    free_before, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    free_after, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() <= before
    assert torch.cuda.max_memory_allocated() == before  # the peak never rose above the start
    assert abs(free_before - free_after) < 2 * 1024 * 1024


def test_last_round_with_one_idle_cu():
    """units = CUs - 1: splitting would put every tail on the one idle CU, so
    the fused launch keeps the last round whole.  Parity, and a time of the
    order of one unit's work (not one tail per unit in a row).  20 x 12 has
    five key tiles, so it takes the split-grid form."""
    cus = _cus()
    H, W = 20, 12
    assert not _small_grid(H, W)
    d = G.make("tiny", B=1, heads=cus - 1, H=H, W=W)
    ref, _, _ = G.oracle_full(d)
    _check(f"{cus - 1} units", np.abs(G.f64(_fused(d)) - ref))
    g = G.to_dev(d)
    ws = torch.empty(_ws_bytes(H, W), dtype=torch.uint8, device="cuda")
    call = lambda: rp.relpos_attn_fused(g["q"], g["k"], g["v"], g["rel_pos_h"], g["rel_pos_w"], H, W,
                                        d["scale"], workspace=ws)
    call()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(5):
        call()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 5
    print(f"[fused] {cus - 1} units of 5 tiles: {ms * 1e3:.1f} us", flush=True)
    assert ms < 1.0


@pytest.mark.parametrize("H,W", [(72, 16), (76, 16), (68, 32)])
def test_rel_h_rows_at_the_lds_limit(H, W):
    """H = 72 fills a 160 KB LDS exactly (rel_h rows in LDS), H = 76 does not
    (rows in the workspace slot); both calls, every output."""
    d = G.make("tiny", B=1, heads=2, H=H, W=W)
    ref, _, _ = G.oracle_full(d)
    _check(f"fused {H}x{W}", np.abs(G.f64(_fused(d)) - ref))
    two, _, _ = G.gpu_run(d)
    _check(f"two calls {H}x{W}", np.abs(G.f64(two) - ref))


# ---- small grids: the 16-query kernel with its bias rows in LDS (no workspace) ----

SMALL = [(1, 1), (1, 7), (5, 3), (7, 9), (14, 14), (16, 16), (16, 8), (4, 32), (8, 32), (2, 17), (13, 11),
         (16, 1), (8, 31)]


@pytest.mark.parametrize("H,W", SMALL)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_small_grid_fused_full(H, W, dtype):
    """Every output against the oracle; no workspace is passed, and the
    result equals the two-call path's within the bar and does not change
    when a (filled) workspace is given, which the call does not read."""
    assert _small_grid(H, W) and _ws_bytes(H, W) == 0
    d = G.make("tiny", seed=H * 53 + W, B=2, heads=3, H=H, W=W, dtype=dtype)
    print(f"[fused] small grid {H}x{W} {dtype}", flush=True)
    ref, _, _ = G.oracle_full(d)
    out = _fused(d)
    _check(f"small {H}x{W} {dtype}", np.abs(G.f64(out) - ref))
    two, _, _ = G.gpu_run(d)
    assert (out - two).abs().max().item() <= G.MAX_ABS
    ws = torch.full((4096,), 0xff, dtype=torch.uint8, device="cuda")
    assert torch.equal(out, _fused(d, ws))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_small_grid_fused_half_output(dtype):
    d = G.make("tiny", dtype=dtype, B=2, heads=2, H=14, W=14)
    out = _fused(d, out_dtype=d["q"].dtype)
    assert out.dtype == d["q"].dtype
    ref, _, _ = G.oracle_full(d)
    err = np.abs(G.f64(out) - ref)
    ulp = 2.0 ** (-8 if dtype == "bf16" else -11)
    assert (err <= G.MAX_ABS + ulp * np.abs(ref)).all(), dtype
    print(f"[fused] small 14x14 out={dtype}: max={err.max():.3e} mean={err.mean():.3e}", flush=True)

