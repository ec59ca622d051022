"""librelpos: attention with a decomposed relative-position bias on MI355X (gfx950).

The compute lives in hand-written HIP kernels behind a C ABI (``librelpos.so``,
declared in ``include/relpos.h``).  This package is a thin ctypes binding with the
same names; it only marshals torch tensors (device memory) and the current stream.
"""

__all__ = ["relpos_build", "relpos_attn_fwd", "relpos_attn_fused", "attn_config", "workspace_bytes",
           "fused_workspace_bytes", "status_string",
           "abi_version", "library_path"]


def __getattr__(name):
    # The binding is imported lazily so that ``inputs`` can be used without the
    # HIP library (for example by the CPU test-suite).
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
