"""Paged-KV-cache decode attention for MI355X (gfx950).

The compute path is ``libpkv.so`` (hand-written HIP kernels behind a C ABI,
see ``include/pkv.h``); this package is a thin ctypes binding over it that only
marshals torch tensors (device pointers, sizes, the current stream).  There is
no CPU fallback: calling a binding without the built library raises.
"""

from ._lib import (PKVError, load_library, paged_attn_decode,  # noqa: F401
                   paged_attn_decode_multi, paged_attn_decode_multi_workspace_size,
                   paged_attn_decode_shared, paged_attn_decode_shared_workspace_size,
                   paged_attn_decode_workspace_size, paged_check_inputs, paged_copy_blocks,
                   paged_decode_step, paged_decode_step_static, paged_kv_write,
                   library_path)

__all__ = ["PKVError", "load_library", "library_path", "paged_kv_write",
           "paged_attn_decode", "paged_attn_decode_workspace_size", "paged_decode_step",
           "paged_decode_step_static",
           "paged_copy_blocks", "paged_attn_decode_multi", "paged_attn_decode_multi_workspace_size",
           "paged_attn_decode_shared", "paged_attn_decode_shared_workspace_size",
           "paged_check_inputs"]
