"""fp64 CPU oracle for paged decode attention and the KV append.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.
"""

from .paged_attention import (DTYPES, copy_blocks, gather_rows,  # noqa: F401
                              paged_attn_decode, paged_kv_write, physical_slot, to_f64)
