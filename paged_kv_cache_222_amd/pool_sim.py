"""Pool-utilisation simulation on the native block pool.

Requests arrive over time and grow token by token in a pool of fixed-size
blocks ("Serving", §23.4 Paged Attention, and its widget: 96 blocks, eight
requests; reserving each maximum lets only four run, paging lets every
request run on arrival).  Each policy draws its blocks from a native
pa_block_pool:

* ``"reserve"``: a request takes ceil(max_len / block_size) blocks when it
  starts and keeps them to the end (its worst case, as one contiguous
  reservation would);
* ``"paged"``: a request takes ceil(prompt / block_size) blocks when it
  starts and one more each time its tokens cross a block boundary.

Request i arrives at step ``arrivals[i]`` with ``prompt_lens[i]`` tokens and
gains one token per step while it runs, until it holds ``final_lens[i]``;
then it finishes and releases its blocks.  Waiting requests start in arrival
order as soon as their blocks are available.
"""

from __future__ import annotations

from . import _binding as B


def simulate(arrivals, prompt_lens, final_lens, n_blocks, block_size, policy,
             max_len=None):
    """Returns per-request start and finish steps, the number of running
    requests at each step, the mean utilisation (tokens stored / token
    capacity of the blocks held) and each request's block ids."""
    if policy not in ("reserve", "paged"):
        raise ValueError(policy)
    pool = B.pa_pool_create(n_blocks)
    n = len(arrivals)
    blocks = [[] for _ in range(n)]
    tokens = [0] * n
    start = [None] * n
    finish = [None] * n
    running, waiting, trace = [], [], []
    util_num = util_den = 0
    need_res = -(-max_len // block_size) if max_len else None
    step = 0
    while any(f is None for f in finish):
        waiting += [i for i in range(n) if arrivals[i] == step]
        while waiting:
            i = waiting[0]
            need = need_res if policy == "reserve" else -(-prompt_lens[i] // block_size)
            if need > B.pa_pool_available(pool):
                break
            waiting.pop(0)
            blocks[i] = list(B.pa_pool_alloc(pool, need))
            tokens[i] = prompt_lens[i]
            start[i] = step
            running.append(i)
        trace.append(len(running))
        for i in running:
            util_num += tokens[i]
            util_den += len(blocks[i]) * block_size
        for i in list(running):
            if tokens[i] >= final_lens[i]:
                finish[i] = step
                B.pa_pool_release(pool, blocks[i])
                running.remove(i)
                continue
            tokens[i] += 1
            if policy == "paged" and tokens[i] > len(blocks[i]) * block_size:
                blocks[i] += list(B.pa_pool_alloc(pool, 1))
        step += 1
    return {"start": start, "finish": finish, "running": trace,
            "utilisation": util_num / util_den if util_den else 0.0,
            "blocks": [[int(b) for b in bl] for bl in blocks]}
