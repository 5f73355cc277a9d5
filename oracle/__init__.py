"""fp64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Shares no code with
the HIP library or its Python binding.
"""

from .paged_attention import (  # noqa: F401
    kv_cache_bytes,
    oracle_cache_write,
    oracle_copy_blocks,
    oracle_decode,
    oracle_decode_multi,
    oracle_decode_row,
    oracle_merge,
    oracle_partitions,
    to_f64,
)
