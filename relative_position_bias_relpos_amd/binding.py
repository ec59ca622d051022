"""ctypes binding of librelpos (include/relpos.h), same names as the C calls.

Argument marshalling only: every step of the computation runs in the HIP
kernels.  Torch provides device memory (the output buffers are allocated here
with torch, O(N*(D+H+W)) bytes) and the stream (torch's current stream).  There
is no fallback: if the library is missing or a call fails, this raises.
"""

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librelpos.so")

RELPOS_BF16, RELPOS_FP16, RELPOS_FP32 = 0, 1, 2
_DT = {torch.bfloat16: RELPOS_BF16, torch.float16: RELPOS_FP16, torch.float32: RELPOS_FP32}

_lock = threading.Lock()
_lib = None
# Raw handle of torch's current stream on a device (an integer); the public
# torch.cuda.current_stream() builds a Stream object per call (about 1.9 us).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


class RelposError(RuntimeError):
    def __init__(self, call, status, message):
        super().__init__(f"{call} failed: status {status} ({message})")
        self.status = status


def library_path():
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m relative_position_bias_relpos_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        i64, vp, f32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
        lib.relpos_build.restype = i32
        lib.relpos_build.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
        lib.relpos_attn_fwd.restype = i32
        lib.relpos_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, i32, vp]
        lib.relpos_status_string.restype = ctypes.c_char_p
        lib.relpos_status_string.argtypes = [i32]
        lib.relpos_abi_version.restype = i32
        lib.relpos_abi_version.argtypes = []
        lib.relpos_attn_fwd_ws.restype = i32
        lib.relpos_attn_fwd_ws.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, i32,
                                           vp, i64, vp]
        lib.relpos_attn_workspace_bytes.restype = i64
        lib.relpos_attn_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i32]
        lib.relpos_attn_fused.restype = i32
        lib.relpos_attn_fused.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, i32,
                                          vp, i64, vp]
        lib.relpos_attn_fused_noalloc.restype = i32
        lib.relpos_attn_fused_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, i32,
                                                  vp]
        lib.relpos_fused_workspace_bytes.restype = i64
        lib.relpos_fused_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i32]
        lib.relpos_attn_config.restype = i32
        lib.relpos_attn_config.argtypes = [i64, i64, i64, i64, i32, i32, i32]
        lib.relpos_attn_fwd_cfg.restype = i32
        lib.relpos_attn_fwd_cfg.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32, i32,
                                            i32, vp, i64, vp]
        _lib = lib
        return lib


def status_string(status):
    return _load().relpos_status_string(int(status)).decode()


def abi_version():
    return _load().relpos_abi_version()


def attn_config(B, heads, H, W, dtype, cu_count, with_workspace=False):
    """Launch configuration the attention call uses for this problem on a
    device with `cu_count` compute units (0: 8-wave workgroups, 1: 4-wave,
    3: 16-query waves, 5: key range split, only with a workspace, 6: 12-wave
    workgroups of 192 queries); host-only."""
    c = _load().relpos_attn_config(int(B), int(heads), int(H), int(W), _DT[dtype], int(cu_count),
                                   1 if with_workspace else 0)
    if c < 0:
        raise ValueError("sizes or dtype out of range for relpos_attn_fwd")
    return c


def workspace_bytes(B, heads, H, W, dtype, cu_count):
    """Bytes of workspace relpos_attn_fwd_ws needs (0: no split, none used)."""
    n = _load().relpos_attn_workspace_bytes(int(B), int(heads), int(H), int(W), _DT[dtype], int(cu_count))
    if n < 0:
        raise ValueError("sizes or dtype out of range for relpos_attn_fwd")
    return n


def fused_workspace_bytes(B, heads, H, W, dtype, cu_count):
    """Bytes of workspace relpos_attn_fused needs on `cu_count` compute units."""
    n = _load().relpos_fused_workspace_bytes(int(B), int(heads), int(H), int(W), _DT[dtype], int(cu_count))
    if n < 0:
        raise ValueError("sizes or dtype out of range for relpos_attn_fused")
    return n


_cus = {}
_workspaces = {}  # (device index, stream handle) -> uint8 scratch tensor of relpos_attn_fused


def _cu_count(device):
    if device.index not in _cus:
        _cus[device.index] = torch.cuda.get_device_properties(device).multi_processor_count
    return _cus[device.index]


def _cached_workspace(device, stream, nbytes):
    """relpos_attn_fused's scratch workspace for one (device, stream): calls on
    one stream never overlap, so it is reused, grown when a larger problem
    needs more, and kept until release_workspaces()."""
    key = (device.index, stream)
    with _lock:
        ws = _workspaces.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
            _workspaces[key] = ws
        return ws


def cached_workspace_bytes():
    """Bytes held by the workspaces relpos_attn_fused(workspace="auto") keeps."""
    with _lock:
        return sum(w.numel() for w in _workspaces.values())


def release_workspaces():
    """Drop the cached relpos_attn_fused workspaces (the memory returns to
    torch's allocator once the work queued on their streams has finished)."""
    with _lock:
        _workspaces.clear()


def _ptr(t):
    # an integer for the c_void_p parameters (None passes NULL)
    return t.data_ptr() if t is not None else None


def _stream(t):
    """Handle (integer) of torch's current stream on t's device."""
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(call, status):
    if status != 0:
        raise RelposError(call, status, status_string(status))


def _dims(q, H, W):
    if q.dim() != 4:
        raise ValueError("q must be [B, heads, H*W, D]")
    B, nh, N, D = q.shape
    if N != H * W:
        raise ValueError(f"q has {N} tokens but H*W = {H * W}")
    return B, nh, D


def _need(t, name, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def relpos_build(q, rel_pos_h, rel_pos_w, H, W, rel_h=None, rel_w=None):
    """rel_h [B,heads,H*W,H], rel_w [B,heads,H*W,W] (fp32) from q and the tables."""
    lib = _load()
    B, nh, D = _dims(q, H, W)
    _need(q, "q")
    _need(rel_pos_h, "rel_pos_h", q.dtype)
    _need(rel_pos_w, "rel_pos_w", q.dtype)
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("q must be bfloat16 or float16")
    if rel_h is None:
        rel_h = torch.empty((B, nh, H * W, H), dtype=torch.float32, device=q.device)
    if rel_w is None:
        rel_w = torch.empty((B, nh, H * W, W), dtype=torch.float32, device=q.device)
    _need(rel_h, "rel_h", torch.float32)
    _need(rel_w, "rel_w", torch.float32)
    st = lib.relpos_build(_ptr(q), _ptr(rel_pos_h), _ptr(rel_pos_w), _ptr(rel_h), _ptr(rel_w),
                          B, nh, H, W, D, _DT[q.dtype], _stream(q))
    _check("relpos_build", st)
    return rel_h, rel_w


def relpos_attn_fwd(q, k, v, rel_h, rel_w, H, W, scale, out=None, out_dtype=torch.float32,
                    workspace=None, config=None):
    """out [B,heads,H*W,D] = softmax(scale*q.k + rel_h[:, j/W] + rel_w[:, j%W]) @ v.

    workspace: None (default) calls relpos_attn_fwd, which needs no scratch
    memory; a uint8 device tensor calls relpos_attn_fwd_ws, which may then
    split the key range of the last round of query units across idle compute
    units (workspace_bytes() says how much it needs; 0 means no split).
    config: None for the library's own choice of launch configuration, or one
    of the configurations include/relpos.h lists (relpos_attn_fwd_cfg; for
    measurements and tests).
    """
    lib = _load()
    B, nh, D = _dims(q, H, W)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
        if t.shape != q.shape:
            raise ValueError(f"{name} must have the shape of q")
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("q, k, v must be bfloat16 or float16")
    _need(rel_h, "rel_h", torch.float32)
    _need(rel_w, "rel_w", torch.float32)
    if rel_h.shape != (B, nh, H * W, H) or rel_w.shape != (B, nh, H * W, W):
        raise ValueError("rel_h/rel_w must be [B, heads, H*W, H] and [B, heads, H*W, W]")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _need(out, "out")
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    if workspace is not None and not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be None or a device tensor")
    ws_ptr = _ptr(workspace)
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if config is not None:
        st = lib.relpos_attn_fwd_cfg(_ptr(q), _ptr(k), _ptr(v), _ptr(rel_h), _ptr(rel_w), _ptr(out),
                                     B, nh, H, W, D, float(scale), _DT[q.dtype], _DT[out.dtype],
                                     int(config), ws_ptr, ws_len, _stream(q))
        _check("relpos_attn_fwd_cfg", st)
    elif workspace is None:
        st = lib.relpos_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(rel_h), _ptr(rel_w), _ptr(out),
                                 B, nh, H, W, D, float(scale), _DT[q.dtype], _DT[out.dtype], _stream(q))
        _check("relpos_attn_fwd", st)
    else:
        st = lib.relpos_attn_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(rel_h), _ptr(rel_w), _ptr(out),
                                    B, nh, H, W, D, float(scale), _DT[q.dtype], _DT[out.dtype],
                                    ws_ptr, ws_len, _stream(q))
        _check("relpos_attn_fwd_ws", st)
    return out


def _fused_operands(q, k, v, rel_pos_h, rel_pos_w, H, W, out, out_dtype):
    B, nh, D = _dims(q, H, W)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype)
        if t.shape != q.shape:
            raise ValueError(f"{name} must have the shape of q")
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("q, k, v must be bfloat16 or float16")
    _need(rel_pos_h, "rel_pos_h", q.dtype)
    _need(rel_pos_w, "rel_pos_w", q.dtype)
    if tuple(rel_pos_h.shape) != (2 * H - 1, D) or tuple(rel_pos_w.shape) != (2 * W - 1, D):
        raise ValueError("rel_pos_h/rel_pos_w must be [2H-1, D] and [2W-1, D]")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _need(out, "out")
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    return B, nh, D, out


def relpos_attn_fused(q, k, v, rel_pos_h, rel_pos_w, H, W, scale, out=None, out_dtype=torch.float32,
                      workspace="auto"):
    """relpos_build and relpos_attn_fwd in one launch: out [B,heads,H*W,D] from
    q, k, v and the tables, without rel_h/rel_w tensors.

    workspace: "auto" (default) uses a scratch workspace cached per (device,
    stream) until release_workspaces(), or none where fused_workspace_bytes()
    is 0 (grids of at most 32 x 32 with at most four key tiles); a uint8
    device tensor of at least fused_workspace_bytes() is used as given.
    """
    lib = _load()
    B, nh, D, out = _fused_operands(q, k, v, rel_pos_h, rel_pos_w, H, W, out, out_dtype)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto" or a tensor')
        need = fused_workspace_bytes(B, nh, H, W, q.dtype, _cu_count(q.device))
        workspace = _cached_workspace(q.device, _stream(q), need) if need > 0 else None
    elif not isinstance(workspace, torch.Tensor):
        raise TypeError('workspace must be "auto" or a tensor')
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.relpos_attn_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(rel_pos_h), _ptr(rel_pos_w), _ptr(out),
                               B, nh, H, W, D, float(scale), _DT[q.dtype], _DT[out.dtype],
                               _ptr(workspace), ws_bytes, _stream(q))
    _check("relpos_attn_fused", st)
    return out


def relpos_attn_fused_noalloc(q, k, v, rel_pos_h, rel_pos_w, H, W, scale, out):
    """relpos_attn_fused on the library's fixed per-device scratch array: the
    call allocates nothing (out must be given).  Calls that may overlap on one
    device (several streams or threads) race on the shared array."""
    lib = _load()
    if out is None:
        raise ValueError("out must be given: relpos_attn_fused_noalloc allocates nothing")
    B, nh, D, out = _fused_operands(q, k, v, rel_pos_h, rel_pos_w, H, W, out, None)
    st = lib.relpos_attn_fused_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(rel_pos_h), _ptr(rel_pos_w), _ptr(out),
                                       B, nh, H, W, D, float(scale), _DT[q.dtype], _DT[out.dtype], _stream(q))
    _check("relpos_attn_fused_noalloc", st)
    return out
