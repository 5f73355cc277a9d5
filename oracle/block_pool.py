"""Plain reference for the host-side block pool, prefix cache and the
pool-utilisation simulation.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests,
the smoke check and the benchmark's CPU-baseline leg, never by the product
path, and sharing no code with it.

What it follows:

* Paging ("Serving", §23.4 Paged Attention): the cache lives in fixed-size
  blocks handed out as a sequence grows; sequences sharing a prefix can share
  its blocks.  The §23.4 widget: a pool of 96 blocks serving eight requests
  that arrive over time and grow token by token; reserving each request's
  maximum lets only four run, paging lets every request run on arrival.
* Prefix caching by block hashes (the prompt-caching articles on the
  pagedattention tag page): a full block is named by a hash of its tokens
  chained with the previous block's hash, so reuse needs an identical prefix
  and one changed token invalidates every later block.
* FNV-1a, 64-bit (Fowler, Noll, Vo): start from the offset basis
  14695981039346656037; for each byte, xor it in, then multiply by the prime
  1099511628211 modulo 2^64.

Readings where the pages are silent (the hash function and its byte layout,
the allocation and reuse order, the widget's request sizes) are the ones the
library documents; they are restated at each function.
"""

from __future__ import annotations

MASK64 = (1 << 64) - 1
FNV_OFFSET = 14695981039346656037
FNV_PRIME = 1099511628211


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """FNV-1a over ``data`` starting from ``h``."""
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_hashes(tokens, block_size: int, parent: int = 0) -> list:
    """Chained hashes of the full blocks of ``tokens``: block i hashes the 8
    little-endian bytes of the previous hash (``parent`` before block 0)
    followed by its token ids as 4-byte little-endian integers."""
    out = []
    h = parent
    for i in range(len(tokens) // block_size):
        data = h.to_bytes(8, "little")
        for t in tokens[i * block_size:(i + 1) * block_size]:
            data += (int(t) & 0xFFFFFFFF).to_bytes(4, "little")
        h = fnv1a64(data)
        out.append(h)
    return out


class OraclePool:
    """Reference counts, a free set and a hash -> block cache.

    A fresh block is the lowest-numbered free block without a cached hash;
    when there is none, the cached free block released longest ago is reused
    and its hash dropped.  A block whose count falls to zero is free; a cached
    one stays findable by its hash until reused."""

    def __init__(self, n_blocks: int):
        self.n = n_blocks
        self.ref = [0] * n_blocks
        self.hash_of = {}          # block -> hash (cached blocks)
        self.block_of = {}         # hash -> block
        self.release_order = []    # cached free blocks, oldest release first

    def available(self) -> int:
        free = [b for b in range(self.n) if self.ref[b] == 0]
        return len(free)

    def _fresh(self) -> int:
        plain = [b for b in range(self.n)
                 if self.ref[b] == 0 and b not in self.hash_of]
        if plain:
            b = min(plain)
        else:
            b = self.release_order.pop(0)
            del self.block_of[self.hash_of.pop(b)]
        self.ref[b] = 1
        return b

    def alloc(self, n: int):
        if n > self.available():
            return None
        return [self._fresh() for _ in range(n)]

    def fork(self, ids) -> bool:
        if any(not (0 <= b < self.n) or self.ref[b] < 1 for b in ids):
            return False
        for b in ids:
            self.ref[b] += 1
        return True

    def release(self, ids) -> bool:
        need = {}
        for b in ids:
            need[b] = need.get(b, 0) + 1
        if any(not (0 <= b < self.n) or self.ref[b] < c for b, c in need.items()):
            return False
        for b in ids:
            self.ref[b] -= 1
            if self.ref[b] == 0 and b in self.hash_of:
                self.release_order.append(b)
        return True

    def map_prefix(self, hashes):
        """(ids, n_hit) for a request's full blocks, or None if the fresh
        blocks are not available (then nothing changes)."""
        hit = 0
        while hit < len(hashes) and hashes[hit] in self.block_of:
            hit += 1
        reused = [self.block_of[h] for h in hashes[:hit]]
        free_reused = sum(1 for b in reused if self.ref[b] == 0)
        if len(hashes) - hit > self.available() - free_reused:
            return None
        for b in reused:
            if self.ref[b] == 0:
                self.release_order.remove(b)
            self.ref[b] += 1
        ids = list(reused)
        for h in hashes[hit:]:
            b = self._fresh()
            ids.append(b)
            if h not in self.block_of:
                self.hash_of[b] = h
                self.block_of[h] = b
        return ids, hit


def simulate(arrivals, prompt_lens, final_lens, n_blocks, block_size,
             policy, max_len=None):
    """Requests in a pool of ``n_blocks`` blocks of ``block_size`` tokens.

    Request i arrives at step ``arrivals[i]`` with ``prompt_lens[i]`` tokens
    and gains one token per step while it runs, until it holds
    ``final_lens[i]`` tokens; then it finishes and frees its blocks.  Waiting
    requests start in arrival order as soon as they fit:

    * ``"reserve"``: a request holds ceil(max_len / block_size) blocks from
      start to finish (its worst case, in one piece);
    * ``"paged"``: a request holds ceil(tokens / block_size) blocks, taking a
      new block when its tokens cross a block boundary.

    Returns per-request start and finish steps, the number running at every
    step, and the mean utilisation (tokens stored / token capacity of the
    blocks held)."""
    n = len(arrivals)
    cap = [0] * n                 # blocks held
    tokens = [0] * n
    start = [None] * n
    finish = [None] * n
    free = n_blocks
    running, waiting = [], []
    step = 0
    trace = []
    util_num = util_den = 0
    need_res = -(-max_len // block_size) if max_len else None
    while any(f is None for f in finish):
        for i in range(n):
            if arrivals[i] == step:
                waiting.append(i)
        # start waiting requests in arrival order while they fit
        while waiting:
            i = waiting[0]
            need = need_res if policy == "reserve" else -(-prompt_lens[i] // block_size)
            if need > free:
                break
            waiting.pop(0)
            free -= need
            cap[i] = need
            tokens[i] = prompt_lens[i]
            start[i] = step
            running.append(i)
        trace.append(len(running))
        for i in running:
            util_num += tokens[i]
            util_den += cap[i] * block_size
        # every running request gains a token (or finishes)
        for i in list(running):
            if tokens[i] >= final_lens[i]:
                finish[i] = step
                free += cap[i]
                cap[i] = 0
                running.remove(i)
                continue
            tokens[i] += 1
            if policy == "paged" and tokens[i] > cap[i] * block_size:
                if free == 0:
                    raise RuntimeError("pool exhausted")
                free -= 1
                cap[i] += 1
        step += 1
    return {"start": start, "finish": finish, "running": trace,
            "utilisation": util_num / util_den if util_den else 0.0}
