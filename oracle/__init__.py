"""fp64 CPU oracle for paged decode attention (one or several query tokens per
sequence), the KV append and the copy-on-write block copy.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.
"""

from .paged_attention import (DTYPES, copy_blocks, gather_rows,  # noqa: F401
                              paged_attn_decode, paged_attn_decode_multi, paged_kv_write,
                              physical_slot, query_context_len, to_f64)
