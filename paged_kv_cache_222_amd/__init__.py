"""Paged KV-cache decode attention for MI355X (gfx950).

The compute lives in ``libpa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/pa.h``); this package holds its thin Python binding, the
build step and the seeded synthetic workloads used by tests and benchmarks.
"""
