"""Plain reference for the host-side block pool, prefix cache and the
pool-utilisation simulation.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests,
the smoke check and the benchmark's CPU-baseline leg, never by the product
path, and sharing no code with it.

What it follows:

* Paging ("Serving", §23.4 Paged Attention): cache memory is handed out in
  fixed-size blocks as sequences grow, and a block can be shared by the
  sequences whose prefix it holds.  The section's widget contrasts the two
  policies on a 96-block pool and eight requests arriving over time: with
  worst-case reservations four requests at most hold blocks at once, while
  with paging none of them waits.
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


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def simulate(arrivals, prompt_lens, final_lens, n_blocks, block_size,
             policy, max_len=None):
    """Requests in a pool of ``n_blocks`` blocks of ``block_size`` tokens,
    worked out from each request's timeline rather than step by step.

    Request i arrives at step ``arrivals[i]`` with ``prompt_lens[i]`` tokens
    and, once started at step s_i, holds ``prompt_lens[i] + (t - s_i)``
    tokens at step t until it holds ``final_lens[i]``: it finishes at
    f_i = s_i + final_lens[i] - prompt_lens[i] and frees its blocks after
    that step is counted.  Blocks held at step t ("Serving", section 23.4:
    under paging a request gets one more block each time its tokens outgrow
    the blocks it holds; under reservation it claims its worst case when it
    starts):

    * ``"reserve"``: ceil(max_len / block_size) for every step of its life;
    * ``"paged"``: ceil(tokens(t) / block_size).

    Start steps follow from one recurrence on the free blocks: requests
    start in arrival order (ties by index); request i starts at the first
    step t >= arrivals[i], not before the request ahead of it, at which its
    first step's blocks fit in n_blocks minus the blocks held at t by the
    requests already started with s_j <= t <= f_j.  Utilisation sums, over
    every step and running request, the tokens stored and the capacity of
    the blocks held (blocks * block_size).  Raises RuntimeError when a
    request could never start or the paged pool would overflow."""
    n = len(arrivals)
    bs = block_size
    life = [final_lens[i] - prompt_lens[i] for i in range(n)]

    def held(i, s, t):
        if policy == "reserve":
            return _ceil_div(max_len, bs)
        return _ceil_div(prompt_lens[i] + (t - s), bs)

    order = sorted(range(n), key=lambda i: (arrivals[i], i))
    start = [None] * n
    t = 0
    for k, i in enumerate(order):
        need = held(i, 0, 0)
        if need > n_blocks:
            raise RuntimeError("a request needs more blocks than the pool has")
        t = max(t, arrivals[i])
        while True:
            in_use = sum(held(j, start[j], t) for j in order[:k]
                         if start[j] <= t <= start[j] + life[j])
            if need <= n_blocks - in_use:
                break
            t += 1
        start[i] = t
    finish = [start[i] + life[i] for i in range(n)]
    n_steps = max(finish) + 1 if n else 0
    running, tok, cap = [], 0, 0
    for t in range(n_steps):
        live = [i for i in range(n) if start[i] <= t <= finish[i]]
        blocks = sum(held(i, start[i], t) for i in live)
        if blocks > n_blocks:
            raise RuntimeError("the pool runs out while requests grow")
        running.append(len(live))
        tok += sum(prompt_lens[i] + (t - start[i]) for i in live)
        cap += blocks * bs
    return {"start": start, "finish": finish, "running": running,
            "tokens": tok, "capacity": cap,
            "utilisation": tok / cap if cap else 0.0}
