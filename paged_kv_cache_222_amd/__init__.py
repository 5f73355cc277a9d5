"""Paged KV-cache decode attention for MI355X (gfx950).

The compute lives in ``libpa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/pa.h``); this package holds its thin Python binding, the
build step and the seeded synthetic workloads used by tests and benchmarks.
The library is loaded on first use; a missing library raises.
"""

from ._binding import (  # noqa: F401
    PA_BF16,
    PA_F16,
    PA_F32,
    BlockPool,
    PaError,
    load,
    pa_block_hashes,
    pa_cache_write,
    pa_copy_blocks,
    pa_decode,
    pa_decode_multi,
    pa_decode_partitioned,
    pa_decode_partitioned_vector,
    pa_decode_shared_prefix,
    pa_decode_split,
    pa_decode_step,
    pa_decode_step_noalloc,
    pa_pool_alloc,
    pa_pool_available,
    pa_pool_create,
    pa_pool_destroy,
    pa_pool_fork,
    pa_pool_map_prefix,
    pa_pool_refcount,
    pa_pool_release,
    pa_pool_simulate,
    pa_read_ceiling,
    pa_reduce,
    pa_strerror,
    pa_time_next_attention,
    partition_workspace,
)
