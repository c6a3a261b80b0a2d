"""MI355X-native fused linear cross-entropy (FLCE) and cross-entropy.

The compute path is the HIP library `liblce03.so` (gfx950 kernels behind a C
ABI, declared in include/flce.h). `binding` is a thin ctypes layer over it that
marshals torch tensors into pointers; importing an ABI name from this package
loads the library and fails loudly if it has not been built.
"""

__all__ = [
    "flce_forward_backward", "ce_forward_backward", "ce_shard_stats",
    "flce_shard_stats", "flce_workspace_bytes", "ce_workspace_bytes",
    "flce_check_device_error", "flce_status_string", "flce_plan",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
