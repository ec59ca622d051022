"""C ABI error paths with real device pointers (mirrors the page's review fix that
checks all five tensors are device tensors on one device)."""

import ctypes

import pytest
import torch

from relative_position_bias_relpos_amd import binding as rp

pytestmark = pytest.mark.gpu

BF16, FP16, FP32 = 0, 1, 2
OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_DEVICE, E_ALIAS = 0, 1, 2, 3, 4, 5, 6


def _bufs(H=8, W=8, B=1, nh=2):
    N = H * W
    q, k, v = (torch.randn(B, nh, N, 64, device="cuda").to(torch.bfloat16) for _ in range(3))
    rel_h = torch.zeros(B, nh, N, H, device="cuda")
    rel_w = torch.zeros(B, nh, N, W, device="cuda")
    out = torch.empty(B, nh, N, 64, device="cuda")
    return q, k, v, rel_h, rel_w, out


def _call(ptrs, B=1, nh=2, H=8, W=8, D=64, ind=BF16, outd=FP32):
    lib = rp._load()
    return lib.relpos_attn_fwd(*[ctypes.c_void_p(p) for p in ptrs], B, nh, H, W, D, 0.125, ind, outd,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _ptrs(ts):
    return [t.data_ptr() for t in ts]


def test_ok_then_host_pointer_rejected():
    ts = _bufs()
    assert _call(_ptrs(ts)) == OK
    torch.cuda.synchronize()
    host = torch.empty(1 << 20, dtype=torch.float32)  # ordinary pageable host memory
    for i in range(6):
        p = _ptrs(ts)
        p[i] = host.data_ptr()
        assert _call(p) == E_DEVICE, i
    # the failed query leaves no sticky error: a good call still launches
    assert _call(_ptrs(ts)) == OK
    torch.cuda.synchronize()


def test_claim_larger_than_allocation():
    """A 2048x2048 claim on buffers sized for 8x8 is refused before any launch:
    the claimed ranges of neighbouring buffers overlap (E_ALIAS), and past that
    the allocation-size and LDS-size checks refuse it (E_SHAPE)."""
    ts = list(_bufs())
    assert _call(_ptrs(ts), H=2048, W=2048) in (E_SHAPE, E_ALIAS)


def test_misaligned_and_alias_on_device():
    ts = _bufs()
    p = _ptrs(ts)
    p[0] += 2
    assert _call(p) == E_ALIGN
    p = _ptrs(ts)
    p[5] = p[1]
    assert _call(p) == E_ALIAS


def test_binding_raises():
    q, k, v, rel_h, rel_w, out = _bufs()
    with pytest.raises(ValueError):
        rp.relpos_attn_fwd(q, k, v, rel_h, rel_w, 8, 4, 0.125)  # H*W mismatch
    with pytest.raises(ValueError):
        rp.relpos_attn_fwd(q.cpu(), k, v, rel_h, rel_w, 8, 8, 0.125)
    with pytest.raises(ValueError):
        rp.relpos_attn_fwd(q, k.half(), v, rel_h, rel_w, 8, 8, 0.125)
    q32 = torch.randn(1, 2, 64, 32, device="cuda").to(torch.bfloat16)
    with pytest.raises(rp.RelposError) as ei:
        rp.relpos_attn_fwd(q32, q32, q32, rel_h, rel_w, 8, 8, 0.125)
    assert ei.value.status == E_SHAPE


def test_empty_batch_noop():
    q = torch.empty(0, 2, 64, 64, device="cuda", dtype=torch.bfloat16)
    rel_h = torch.empty(0, 2, 64, 8, device="cuda")
    rel_w = torch.empty(0, 2, 64, 8, device="cuda")
    out = rp.relpos_attn_fwd(q, q, q, rel_h, rel_w, 8, 8, 0.125)
    assert out.shape == (0, 2, 64, 64)
