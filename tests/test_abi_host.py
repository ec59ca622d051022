"""C ABI checks that need no GPU: the library loads, exports every symbol that
include/relpos.h declares, and rejects bad arguments before touching the device.

The validation order documented in the header (sizes, dtypes, scalars, then
NULL, alignment and overlap) means these calls return before any HIP call, so
fake pointer values are safe: they are compared, never dereferenced.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "relpos.h")
LIB = os.path.join(ROOT, "relative_position_bias_relpos_amd", "librelpos.so")

BF16, FP16, FP32 = 0, 1, 2
OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_DEVICE, E_ALIAS, E_LAUNCH, E_HIP, E_VALUE = range(10)


def _declared():
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:relpos_status|const char\*|int64_t|int)\s+(relpos_\w+)\s*\(", text, re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("librelpos.so not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    i64, vp, f32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    lib.relpos_build.restype = i32
    lib.relpos_build.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
    lib.relpos_attn_fwd.restype = i32
    lib.relpos_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, i32, vp]
    lib.relpos_status_string.restype = ctypes.c_char_p
    lib.relpos_status_string.argtypes = [i32]
    return lib


def test_header_declares_the_calls():
    names = set(_declared())
    assert {"relpos_build", "relpos_attn_fwd", "relpos_attn_fwd_ws", "relpos_attn_workspace_bytes",
            "relpos_attn_config", "relpos_attn_fwd_cfg", "relpos_status_string", "relpos_abi_version"} <= names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_abi_version(lib):
    text = open(HEADER).read()
    want = int(re.search(r"#define RELPOS_ABI_VERSION (\d+)", text).group(1))
    assert lib.relpos_abi_version() == want


def test_status_strings(lib):
    seen = set()
    for code in range(10):
        s = lib.relpos_status_string(code)
        assert s and s != b"unknown status"
        seen.add(s)
    assert len(seen) == 10
    assert lib.relpos_status_string(99) == b"unknown status"


P = [0x10000 * (i + 1) for i in range(6)]  # distinct, aligned, never dereferenced


def attn(lib, ptrs=None, B=1, nh=2, H=4, W=4, D=64, scale=0.125, ind=BF16, outd=FP32):
    p = ptrs or P
    return lib.relpos_attn_fwd(*p, B, nh, H, W, D, scale, ind, outd, None)


def build(lib, ptrs=None, B=1, nh=2, H=4, W=4, D=64, ind=BF16):
    p = ptrs or P[:5]
    return lib.relpos_build(*p, B, nh, H, W, D, ind, None)


def test_shape_errors(lib):
    assert attn(lib, D=32) == E_SHAPE
    assert build(lib, D=128) == E_SHAPE
    assert attn(lib, H=0) == E_SHAPE
    assert attn(lib, W=-1) == E_SHAPE
    assert attn(lib, H=5000) == E_SHAPE
    assert attn(lib, H=4096, W=4097) == E_SHAPE
    assert attn(lib, B=-1) == E_SHAPE
    assert attn(lib, B=70000, nh=1) == E_SHAPE
    assert build(lib, B=300, nh=300) == E_SHAPE


def test_dtype_errors(lib):
    assert attn(lib, ind=FP32) == E_DTYPE
    assert attn(lib, ind=7) == E_DTYPE
    assert attn(lib, ind=BF16, outd=FP16) == E_DTYPE
    assert attn(lib, ind=FP16, outd=BF16) == E_DTYPE
    assert build(lib, ind=FP32) == E_DTYPE


def test_scale_must_be_finite(lib):
    assert attn(lib, scale=float("nan")) == E_VALUE
    assert attn(lib, scale=float("inf")) == E_VALUE


def test_scale_rule(lib):
    """0 and any |scale| >= 2^-64 pass the scalar check (the call then stops at
    the misaligned pointer); 0 < |scale| < 2^-64 is E_VALUE."""
    bad = [x + 2 for x in P]
    for scale in (0.0, -0.0, -0.125, 2.0 ** -64, -(2.0 ** -64), 1e30):
        assert attn(lib, ptrs=bad, scale=scale) == E_ALIGN, scale
        assert _fused(lib, ptrs=bad + [0x10000 * 7 + 2], scale=scale) == E_ALIGN, scale
    for scale in (2.0 ** -65, -(2.0 ** -70), 1e-30, 1e-45):
        assert attn(lib, ptrs=bad, scale=scale) == E_VALUE, scale
        assert _fused(lib, ptrs=bad + [0x10000 * 7 + 2], scale=scale) == E_VALUE, scale


def _cfg_call(lib, config, ptrs=None, ws=0, ws_bytes=0, D=64, scale=0.125):
    f = lib.relpos_attn_fwd_cfg
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    f.restype = ctypes.c_int
    f.argtypes = [vp] * 6 + [i64] * 5 + [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, i64, vp]
    p = ptrs or P
    return f(*[vp(x) for x in p], 1, 2, 4, 4, D, scale, BF16, FP32, config, vp(ws), ws_bytes, vp(0))


def test_attn_fwd_cfg_argument_checks(lib):
    bad = [x + 2 for x in P]
    for config in (-1, 0, 1, 3, 5, 6):  # known configurations reach the pointer checks
        assert _cfg_call(lib, config, ptrs=bad) == E_ALIGN, config
    for config in (-2, 2, 4, 7, 1000):
        assert _cfg_call(lib, config, ptrs=bad) == E_VALUE, config
    assert _cfg_call(lib, 0, ptrs=bad, ws_bytes=-1) == E_VALUE
    assert _cfg_call(lib, 0, D=32) == E_SHAPE


def test_empty_batch_is_a_noop(lib):
    assert attn(lib, ptrs=[None] * 6, B=0) == OK
    assert attn(lib, ptrs=[None] * 6, nh=0) == OK
    assert build(lib, ptrs=[None] * 5, B=0) == OK


def test_null_pointers(lib):
    for i in range(6):
        p = list(P)
        p[i] = None
        assert attn(lib, ptrs=p) == E_NULL
    for i in range(5):
        p = list(P[:5])
        p[i] = None
        assert build(lib, ptrs=p) == E_NULL


def test_misaligned(lib):
    for i in range(6):
        p = list(P)
        p[i] += 2
        assert attn(lib, ptrs=p) == E_ALIGN


def test_aliasing(lib):
    p = list(P)
    p[5] = p[0]  # out == q
    assert attn(lib, ptrs=p) == E_ALIAS
    p = list(P)
    p[5] = p[3] + 16  # out inside rel_h
    assert attn(lib, ptrs=p) == E_ALIAS
    p = list(P[:5])
    p[4] = p[3]  # rel_w == rel_h
    assert build(lib, ptrs=p) == E_ALIAS
    p = list(P[:5])
    p[3] = p[0]  # rel_h over q
    assert build(lib, ptrs=p) == E_ALIAS


# ---- launch configuration choice (host-only cost model) ----------------------

def _cfg(lib, B, heads, H, W, dt, cus=256, ws=0):
    lib.relpos_attn_config.restype = ctypes.c_int
    lib.relpos_attn_config.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    return lib.relpos_attn_config(B, heads, H, W, dt, cus, ws)


def _ws_bytes(lib, B, heads, H, W, dt, cus=256):
    lib.relpos_attn_workspace_bytes.restype = ctypes.c_int64
    lib.relpos_attn_workspace_bytes.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_int]
    return lib.relpos_attn_workspace_bytes(B, heads, H, W, dt, cus)


TWELVE = 6


def test_attn_config_on_the_workloads(lib):
    # bf16 with N >= 2048: the 12-wave kernel (192 queries per workgroup, a
    # round at 0.91 * 0.75 * 1.05 = 0.717).
    # 64x64, 12 heads: 1536 blocks of 32 = 256 workgroups, one round (0.717),
    # against 192 8-wave workgroups in one round (0.91).
    assert _cfg(lib, 1, 12, 64, 64, BF16) == TWELVE
    # 48x80, 2x12 heads: 480 workgroups, two rounds (1.43), against 8 waves
    # (360 workgroups, two rounds: 1.82) and 4 waves (720: 1 + 0.77).
    assert _cfg(lib, 2, 12, 48, 80, BF16) == TWELVE
    # 96x96, 2x16 heads: 1536 workgroups, six rounds (4.30), against 5 rounds
    # x 0.91 = 4.55 and 4 + 0.77.
    assert _cfg(lib, 2, 16, 96, 96, BF16) == TWELVE
    # bf16 64x64, 4x12 heads: four 12-wave rounds (2.87) against three 8-wave
    # rounds (2.73).
    assert _cfg(lib, 4, 12, 64, 64, BF16) == 0
    # fp16 64x64, 4x12 heads: 3 rounds each; without a V conversion to share,
    # an 8-wave round counts 0.985 -> 8 waves, by a small margin.  fp16 never
    # takes the 12-wave kernel.
    assert _cfg(lib, 4, 12, 64, 64, FP16) == 0
    assert _cfg(lib, 2, 16, 96, 96, FP16) == 1


def test_attn_config_twelve_wave_limits(lib):
    # bf16 below 2048 keys (fp16 P there) is left to the other kernels:
    # 16x32 grids, 96 heads = 3072 blocks of 32 would be 512 workgroups;
    # 32x32 grids, 12 heads.
    assert _cfg(lib, 1, 96, 16, 32, BF16) != TWELVE
    assert _cfg(lib, 1, 12, 32, 32, BF16) != TWELVE
    # From 2048 keys on: 32x64, 12 heads, 128 workgroups in one round.
    assert _cfg(lib, 1, 12, 32, 64, BF16) == TWELVE
    # More than one round where 8-wave units fill the chip evenly: 64x64 with
    # 16 heads is exactly 256 8-wave workgroups (0.91) against 342 12-wave
    # workgroups (two rounds, 1.43).
    assert _cfg(lib, 1, 16, 64, 64, BF16) == 0


def test_attn_config_rounds_arithmetic(lib):
    # One (b, h) of 256 queries (32x8 grid, 8 key tiles): one 8-wave round
    # (0.91) against two lone 4-wave workgroups (0.77).
    assert _cfg(lib, 1, 1, 32, 8, BF16) == 1
    # 512 heads of 256 queries (32x8 grids): exactly two full 4-wave rounds
    # (1024 workgroups) against two 8-wave rounds at 0.91 (bf16) or 0.985 (fp16).
    assert _cfg(lib, 1, 512, 32, 8, BF16) == 0
    assert _cfg(lib, 1, 512, 32, 8, FP16) == 0
    # fp16 still takes 4 waves where a lone last round decides: one (b, h) of
    # 256 queries, 0.985 against 0.77.
    assert _cfg(lib, 1, 1, 32, 8, FP16) == 1
    # 1024 heads of 128 queries (32x4 grids): an 8-wave workgroup would be
    # half empty (four rounds) against two full 4-wave rounds.
    assert _cfg(lib, 1, 1024, 32, 4, BF16) == 1
    # The CU count enters: on 128 CUs the 64x64 workload needs two 8-wave
    # rounds (1.82) against 384 = 1.5 rounds of 4 waves (1 + 0.77); fp16,
    # for which the 12-wave kernel is not considered, takes 4 waves.
    assert _cfg(lib, 1, 12, 64, 64, FP16, cus=128) == 1
    # bf16: 256 12-wave workgroups on 128 CUs, two rounds (1.43).
    assert _cfg(lib, 1, 12, 64, 64, BF16, cus=128) == 6


def test_attn_config_short_key_loops(lib):
    # At most 4 key tiles of 4x16 cells per unit -> configuration 3, the
    # 16-query kernel: 14x14 windows (4 tiles), the 16x16 grid (4), 8x32 (4).
    assert _cfg(lib, 25, 12, 14, 14, BF16) == 3
    assert _cfg(lib, 1, 2, 16, 16, BF16) == 3
    assert _cfg(lib, 1, 2, 8, 32, FP16) == 3
    assert _cfg(lib, 25, 12, 14, 14, BF16, ws=1) == 3
    # 5 tiles (20x16) and more go to the rounds model.
    assert _cfg(lib, 1, 2, 20, 16, BF16) in (0, 1)


def test_attn_config_rejects_bad_input(lib):
    assert _cfg(lib, 1, 1, 0, 8, BF16) == -1
    assert _cfg(lib, 1, 1, 8, 8, FP32) == -1
    assert _cfg(lib, 1, 1, 8, 8, BF16, cus=0) == -1


def test_attn_config_with_workspace(lib):
    SPLIT = 5
    # 64x64, 12 heads: 192 units of 64 tiles on 256 CUs, no full round; the
    # 64 idle CUs take 3 tails each.  With 6 tiles per segment, s = (3*64 +
    # 2*6) / 4 = 51: head 51 + 6 = 57, tails 3 * (13 + 6) = 57, so
    # 0.91 * 1.06 * (57 + 4) / 64 = 0.919 rounds against 0.91 unsplit and
    # 0.717 for the 12-wave kernel.
    assert _cfg(lib, 1, 12, 64, 64, BF16, ws=1) == TWELVE
    assert _cfg(lib, 1, 12, 64, 64, FP16, ws=1) == 0
    # 48x80, 2x12 heads: 360 units of 60 tiles: one full round, then 104 units
    # cut at s = 30 (k = 1): 0.91 * 1.06 * (1 + (36 + 4) / 60) = 1.61 against
    # 1.77 unsplit, but 1.43 for the 12-wave kernel; fp16 splits.
    assert _cfg(lib, 2, 12, 48, 80, BF16, ws=1) == TWELVE
    assert _cfg(lib, 2, 12, 48, 80, FP16, ws=1) == SPLIT
    # 96x96, 2x16 heads: 1152 units of 144 tiles: 4 rounds, then 128 cut at
    # s = 72: 0.91 * 1.06 * (4 + (78 + 4) / 144) = 4.41 < 4.55, but 4.30 for
    # the 12-wave kernel.  fp16 with 16 heads: 2 rounds + 64 units cut,
    # 0.985 * 1.06 * (2 + 82 / 144) = 2.68 against 2 + 0.77.
    assert _cfg(lib, 2, 16, 96, 96, BF16, ws=1) == TWELVE
    assert _cfg(lib, 1, 16, 96, 96, FP16, ws=1) == SPLIT
    # fp16 64x64, 4x12 heads: 768 units = 3 whole rounds; splitting gains nothing.
    assert _cfg(lib, 4, 12, 64, 64, FP16, ws=1) == 0
    # 16x16, 2 heads: 4 key tiles per unit -> the 16-query kernel, split or not.
    assert _cfg(lib, 1, 2, 16, 16, BF16, ws=1) == 3
    # without a workspace the split is never chosen
    assert _cfg(lib, 1, 16, 96, 96, FP16, ws=0) == 1


def test_workspace_bytes(lib):
    # two piece slots of (256*64 + 2*256) floats per compute unit
    assert _ws_bytes(lib, 1, 16, 96, 96, FP16) == 256 * 2 * (256 * 64 + 512) * 4
    # 64x64, 12 heads on 256 CUs: the 12-wave kernel is chosen -> no workspace
    assert _ws_bytes(lib, 1, 12, 64, 64, BF16) == 0
    assert _ws_bytes(lib, 2, 16, 96, 96, BF16) == 0
    # 64x64, 12 fp16 heads on 128 CUs: one full round of 128 units, then 64
    # units split at tile 32: 0.985 * 1.06 * (1 + (38 + 4) / 64) = 1.73
    # against 1.77.  (bf16: two 12-wave rounds, 1.43.)
    assert _cfg(lib, 1, 12, 64, 64, FP16, cus=128, ws=1) == 5
    assert _ws_bytes(lib, 1, 12, 64, 64, FP16, cus=128) == 128 * 2 * (256 * 64 + 512) * 4
    assert _cfg(lib, 1, 12, 64, 64, BF16, cus=128, ws=1) == 6
    assert _ws_bytes(lib, 1, 12, 64, 64, BF16, cus=128) == 0
    # 16x32 grid, 150 heads, 128 CUs: 300 units of 8 tiles, 2 rounds + 44
    # split at tile 4: 0.91 * 1.06 * (2 + (10 + 4) / 8) = 3.62; three 8-wave
    # rounds (2.73) beat 2 + 0.77 4-wave rounds.
    assert _cfg(lib, 1, 150, 16, 32, BF16, cus=128, ws=1) == 0
    assert _ws_bytes(lib, 1, 150, 16, 32, BF16, cus=128) == 0
    # no split chosen -> 0; bad input -> -1
    assert _ws_bytes(lib, 4, 12, 64, 64, FP16) == 0
    assert _ws_bytes(lib, 1, 12, 64, 64, FP32) == -1
    assert _ws_bytes(lib, 1, 12, 64, 64, BF16, cus=0) == -1


def test_attn_fwd_ws_rejects_negative_workspace_size(lib):
    f = lib.relpos_attn_fwd_ws
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    f.restype = ctypes.c_int
    f.argtypes = [vp] * 6 + [i64] * 5 + [ctypes.c_float, ctypes.c_int, ctypes.c_int, vp, i64, vp]
    fake = [vp(0x100000 * (i + 1)) for i in range(6)]
    assert f(*fake, 1, 1, 8, 8, 64, 0.125, BF16, FP32, vp(0x900000), -1, vp(0)) == E_VALUE
    # the size checks still come first
    assert f(*fake, 1, 1, 8, 8, 32, 0.125, BF16, FP32, vp(0x900000), 1024, vp(0)) == E_SHAPE


def test_attn_fwd_grid_limit(lib):
    # 65535 heads on a 4096x4096 grid: 2^18 workgroups of 64 queries per head
    # overflow a 1-D grid -> E_SHAPE before any pointer is looked at.
    vp = ctypes.c_void_p
    assert lib.relpos_attn_fwd(vp(0), vp(0), vp(0), vp(0), vp(0), vp(0), 1, 65535, 4096, 4096, 64,
                               0.125, BF16, FP32, vp(0)) == E_SHAPE


# ---- relpos_attn_fused (host-side checks) ---------------------------------------

def _fused(lib, ptrs=None, B=1, nh=2, H=4, W=4, D=64, scale=0.125, ind=BF16, outd=FP32, ws_bytes=1 << 30):
    f = lib.relpos_attn_fused
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    f.restype = ctypes.c_int
    f.argtypes = [vp] * 6 + [i64] * 5 + [ctypes.c_float, ctypes.c_int, ctypes.c_int, vp, i64, vp]
    p = ptrs or (P + [0x10000 * 7])
    return f(*[vp(x) if x is not None else vp(0) for x in p[:6]], B, nh, H, W, D, scale, ind, outd,
             vp(p[6]) if p[6] is not None else vp(0), ws_bytes, vp(0))


def _fused_ws(lib, B, heads, H, W, dt, cus=256):
    f = lib.relpos_fused_workspace_bytes
    f.restype = ctypes.c_int64
    f.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_int]
    return f(B, heads, H, W, dt, cus)


def test_fused_workspace_bytes(lib):
    # 12-wave fused kernel (bf16, W % 32 == 0, H % 4 == 0, N >= 2048); a slot
    # is 6 blocks x 32 queries x (H + W) floats.  H, W <= 64: units inside one
    # head keep their bias rows in LDS, the others (spanning two heads, or a
    # partial last unit) use one slot per b*heads, or per workgroup of the
    # persistent grid of min(units, CUs) when that is fewer.
    assert _fused_ws(lib, 1, 12, 64, 64, BF16) == 12 * 192 * 128 * 4          # 1.2 MB
    assert _fused_ws(lib, 1, 12, 64, 64, BF16, cus=8) == 8 * 192 * 128 * 4
    assert _fused_ws(lib, 32, 12, 64, 64, BF16) == 256 * 192 * 128 * 4       # 384 heads, 256 CUs
    assert _fused_ws(lib, 1, 1, 64, 64, BF16) == 192 * 128 * 4
    assert _fused_ws(lib, 2, 3, 48, 64, BF16) == 6 * 192 * 112 * 4
    assert _fused_ws(lib, 1, 2, 64, 32, BF16) == 2 * 192 * 96 * 4
    # larger sides: one slot per workgroup of the persistent grid of
    # min(units, CUs) workgroups, units = ceil(B*heads*N/32 / 6).
    # 96x96, 2x16 heads: 1536 units on 256 CUs -> 256 slots
    assert _fused_ws(lib, 2, 16, 96, 96, BF16) == 256 * 192 * 192 * 4
    # one 96x96 head: 48 units -> 48 slots; 64x128 (W > 64): 43 units of 2 heads
    assert _fused_ws(lib, 1, 1, 96, 96, BF16) == 48 * 192 * 192 * 4
    assert _fused_ws(lib, 1, 2, 64, 128, BF16) == 86 * 192 * 192 * 4
    # Otherwise the split-grid kernel: two split pieces and one slot of bias
    # rows (256 queries) per CU.
    piece = 2 * (256 * 64 + 2 * 256)
    # 64x64 fp16: rows padded to 64 + 64 floats per query, 256 queries per slot
    assert _fused_ws(lib, 1, 12, 64, 64, FP16) == 256 * (piece + 256 * 128) * 4
    # 48x80 (W % 32 != 0) -> 48 + 80; 4x48 -> 4 + 48; 20x16 -> 20 + 16
    assert _fused_ws(lib, 2, 12, 48, 80, BF16, cus=128) == 128 * (piece + 256 * 128) * 4
    assert _fused_ws(lib, 1, 1, 4, 48, FP16, cus=8) == 8 * (piece + 256 * 52) * 4
    assert _fused_ws(lib, 1, 1, 20, 16, BF16, cus=1) == (piece + 256 * 36) * 4
    # H, W <= 32 with at most 4 key tiles (4x16 each): the 16-query kernel with
    # the bias rows in LDS, no workspace (14x14 windows, 16x16, 7x9, 8x32, 1x1)
    for H, W in ((14, 14), (16, 16), (7, 9), (8, 32), (1, 1), (4, 32), (16, 8)):
        assert _fused_ws(lib, 25, 12, H, W, BF16) == 0, (H, W)
        assert _fused_ws(lib, 1, 1, H, W, FP16, cus=1) == 0, (H, W)
    # more key tiles, or a side above 32: a workspace
    assert _fused_ws(lib, 1, 1, 17, 16, BF16) > 0   # 5 tiles
    assert _fused_ws(lib, 1, 1, 12, 32, BF16) > 0   # 6 tiles
    assert _fused_ws(lib, 1, 1, 4, 33, BF16) > 0    # W > 32
    assert _fused_ws(lib, 1, 1, 8, 8, FP32) == -1
    assert _fused_ws(lib, 1, 1, 0, 8, BF16) == -1
    assert _fused_ws(lib, 1, 1, 8, 8, BF16, cus=0) == -1


def test_fused_argument_errors(lib):
    # sizes, dtypes and scalars come first (no pointer is looked at)
    assert _fused(lib, D=32) == E_SHAPE
    assert _fused(lib, H=0) == E_SHAPE
    assert _fused(lib, ind=FP32) == E_DTYPE
    assert _fused(lib, ind=BF16, outd=FP16) == E_DTYPE
    assert _fused(lib, scale=float("nan")) == E_VALUE
    assert _fused(lib, ws_bytes=-1) == E_VALUE
    assert _fused(lib, ptrs=[None] * 7, B=0) == OK


def test_fused_is_declared_with_its_workspace_query():
    names = set(_declared())
    assert {"relpos_attn_fused", "relpos_fused_workspace_bytes"} <= names


def test_fused_pointer_errors(lib):
    # 20 x 16 (five key tiles) takes a workspace: all seven pointers are checked.
    base = P + [0x10000 * 7]
    for i in range(7):
        p = list(base)
        p[i] = None
        assert _fused(lib, ptrs=p, H=20, W=16) == E_NULL, i
        p = list(base)
        p[i] += 4
        assert _fused(lib, ptrs=p, H=20, W=16) == E_ALIGN, i
    for H, W in ((20, 16), (4, 4)):
        p = list(base)
        p[5] = p[0]  # out == q
        assert _fused(lib, ptrs=p, H=H, W=W) == E_ALIAS
        p = list(base)
        p[5] = p[3]  # out over rel_pos_h
        assert _fused(lib, ptrs=p, H=H, W=W) == E_ALIAS


def test_fused_small_grid_ignores_workspace(lib):
    # H, W <= 32 with at most four key tiles: the bias rows live in LDS and the
    # workspace argument is not read, so a NULL or unaligned one passes the
    # pointer checks (the call then stops at the planted out == q overlap).
    base = P + [0x10000 * 7]
    for H, W in ((4, 4), (14, 14), (16, 16), (1, 1), (16, 8)):
        for ws in (None, base[6] + 4):
            p = list(base)
            p[6] = ws
            p[5] = p[0]
            assert _fused(lib, ptrs=p, H=H, W=W, ws_bytes=0) == E_ALIAS, (H, W, ws)
        for i in range(6):
            p = list(base)
            p[6] = None
            p[i] = None
            assert _fused(lib, ptrs=p, H=H, W=W, ws_bytes=0) == E_NULL, (H, W, i)


# ---- relpos_attn_fused_noalloc (host-side checks) ----------------------------------

def _noalloc(lib, ptrs=None, B=1, nh=2, H=4, W=4, D=64, scale=0.125, ind=BF16, outd=FP32):
    f = lib.relpos_attn_fused_noalloc
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    f.restype = ctypes.c_int
    f.argtypes = [vp] * 6 + [i64] * 5 + [ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    p = ptrs or P
    return f(*[vp(x) if x is not None else vp(0) for x in p[:6]], B, nh, H, W, D, scale, ind, outd, vp(0))


def _scratch_bytes():
    text = open(HEADER).read()
    m = re.search(r"#define RELPOS_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    return int(m.group(1)) << int(m.group(2))


def test_scratch_size_covers_the_workloads(lib):
    # 96 MiB holds relpos_attn_fused's workspace on 256 CUs for every batch
    # size of the workloads here: the 12-wave kernel's when H + W <= 512, the
    # split-grid kernel's when roundup(H, 4) + roundup(W, 16) <= 252.
    cap = _scratch_bytes()
    assert cap == 96 << 20
    for B, heads, H, W, dt in ((1, 12, 64, 64, BF16), (64, 12, 64, 64, BF16), (4, 12, 64, 64, FP16),
                               (2, 12, 48, 80, BF16), (64, 16, 96, 96, BF16), (25, 12, 14, 14, BF16),
                               (1, 1, 92, 160, BF16), (64, 1, 256, 256, BF16)):
        assert _fused_ws(lib, B, heads, H, W, dt) <= cap, (B, heads, H, W)
    for B, heads, H, W, dt in ((1, 16, 256, 288, BF16), (1, 1, 92, 176, BF16), (1, 1, 128, 128, FP16)):
        assert _fused_ws(lib, B, heads, H, W, dt) > cap, (B, heads, H, W)


def test_noalloc_argument_errors(lib):
    # the checks of relpos_attn_fused, in its order, before any device query
    assert _noalloc(lib, D=32) == E_SHAPE
    assert _noalloc(lib, H=0) == E_SHAPE
    assert _noalloc(lib, ind=FP32) == E_DTYPE
    assert _noalloc(lib, ind=BF16, outd=FP16) == E_DTYPE
    assert _noalloc(lib, scale=float("inf")) == E_VALUE
    assert _noalloc(lib, ptrs=[None] * 6, B=0) == OK
    for i in range(6):
        p = list(P)
        p[i] = None
        assert _noalloc(lib, ptrs=p) == E_NULL, i
        p = list(P)
        p[i] += 4
        assert _noalloc(lib, ptrs=p) == E_ALIGN, i
    p = list(P)
    p[5] = p[1]  # out == k
    assert _noalloc(lib, ptrs=p) == E_ALIAS
