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
    PaError,
    load,
    pa_cache_write,
    pa_copy_blocks,
    pa_decode,
    pa_decode_multi,
    pa_decode_partitioned,
    pa_reduce,
    pa_strerror,
    partition_workspace,
)
