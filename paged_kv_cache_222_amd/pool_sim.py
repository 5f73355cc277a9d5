"""Pool-utilisation simulation: a thin front end of the native
pa_pool_simulate (the loop, the block pool and the accounting are C++ in
libpa; see include/pa.h).

Requests arrive over time and grow token by token in a pool of fixed-size
blocks ("Serving", section 23.4, and its widget of a 96-block pool and eight
requests).  Two policies: ``"reserve"`` holds each request's worst case,
ceil(max_len / block_size) blocks, from start to finish; ``"paged"`` holds
ceil(tokens / block_size) blocks, taking one more as the tokens pass a block
boundary.  Waiting requests start in arrival order when their blocks are
free.
"""

from __future__ import annotations

from . import _binding as B


def simulate(arrivals, prompt_lens, final_lens, n_blocks, block_size, policy,
             max_len=None):
    """Per-request start and finish steps, the number of running requests
    at each step, the utilisation sums (tokens stored, token capacity of
    the blocks held, over every step) and their ratio."""
    return B.pa_pool_simulate(arrivals, prompt_lens, final_lens, n_blocks,
                              block_size, policy, max_len or 0)
