"""KATA (Kernelized Linear Attention Activations) causal forward and decode on MI355X.

The compute path is the HIP library ``libkata.so`` (kernels for gfx950 behind a C
ABI declared in ``include/kata.h``); this package is a thin ctypes binding over it
plus the seeded input generators.  Importing the package does not load the
library; the first call of an entry point does, and fails loudly if it is
missing.
"""
_BINDING_NAMES = (
    "KataError", "abi_version", "backward", "backward_workspace_bytes", "decode_step", "decode_step_decay", "decode_step_delta", "decode_step_factors",
    "forward_decay", "forward_decay_workspace_bytes", "forward_delta", "forward_delta_chunked",
    "forward_delta_chunked_workspace_bytes", "forward_delta_chunked_plan", "forward_factors",
    "forward_factors_workspace_bytes", "feature_map", "flash_forward", "flash_workspace_bytes",
    "forward", "forward_noalloc", "forward_plan", "forward_workspace_bytes", "library_path", "load_library", "NOALLOC_SCRATCH_BYTES",
    "decode_step_packed", "decode_step_decay_packed", "decode_step_delta_packed", "decode_step_factors_packed",
    "state_pack", "state_unpack",
    "PACKED_ROWS",
)

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
