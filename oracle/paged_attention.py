"""fp64 CPU oracle for single-token decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain reference the HIP
path is checked against.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import it; the product path never does,
and this module imports nothing from the product path.

What it computes, and where that comes from:

* The paged layout ("Serving", §23.4 Paged Attention; and the "Paged
  Attention: Managing the KV Cache Like Virtual Memory" summary on the
  inference-serving tag page): the cache lives in fixed-size blocks of
  ``block_size`` token positions, and a per-sequence table maps a position to
  its block.  Position ``t`` of sequence ``b`` lives in physical block
  ``block_table[b, t // block_size]`` at offset ``t % block_size``.
  The pool layout ``[n_blocks, n_kv_heads, block_size, d_head]`` and the flat
  slot ``block * block_size + offset`` are readings: the pages fix neither.
* Decode ("Serving", §23.2 Prefill and Decode): one new query token per
  sequence reads the whole cached K/V of that sequence.  The attention itself
  is the standard scaled dot-product softmax attention the page refers back to
  (its section 12, not among the pages): ``out = softmax(scale * q K^T) V``
  over every cached position ``t < context_len``.
* Grouped-query attention ("Serving", §23.1: LLaMA-3 8B keeps 8 KV heads for
  its 32 query heads): ``G = n_q_heads / n_kv_heads`` query heads share one KV
  head; query head ``h`` reads KV head ``h // G`` (reading: contiguous groups).
* KV-cache size ("Serving", §23.1 The Memory Wall): the product of the two
  (keys and values), layers, KV heads, head width, context, batch and bytes
  per number.

Everything floating point is computed in float64 from the exactly decoded
storage values.  Functions are split into small named steps so a test can
swap one for a deliberately wrong version and see the pins catch it.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Storage decoding (bf16 is carried as uint16 bit patterns)
# ---------------------------------------------------------------------------


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of every stored element."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype in ("f16", "f32"):
        return np.asarray(x).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Small named steps
# ---------------------------------------------------------------------------


def _kv_head(h: int, gqa_group: int) -> int:
    """KV head read by query head ``h``: groups of ``gqa_group`` consecutive
    query heads share one KV head (reading of "Serving", §23.1, GQA)."""
    return h // gqa_group


def _token_location(table_row: np.ndarray, t: np.ndarray, block_size: int):
    """(physical block, offset in block) of positions ``t`` ("Serving", §23.4:
    a per-sequence table maps positions to fixed-size blocks)."""
    return table_row[t // block_size].astype(np.int64), t % block_size


def _gather(pool: np.ndarray, table_row: np.ndarray, kvh: int, start: int,
            stop: int, block_size: int) -> np.ndarray:
    """Rows ``start..stop-1`` of KV head ``kvh`` of one sequence, read through
    its table: ``[stop-start, d_head]`` in storage dtype."""
    t = np.arange(start, stop, dtype=np.int64)
    blk, off = _token_location(table_row, t, block_size)
    return pool[blk, kvh, off, :]


def _logits(q_h: np.ndarray, k_rows: np.ndarray, scale: float) -> np.ndarray:
    """s_t = scale * <q, k_t> for every row ``k_t`` of ``k_rows`` [n, D]."""
    return scale * (k_rows @ q_h)


def _softmax(s: np.ndarray) -> np.ndarray:
    """Numerically stable softmax of a 1-D logit vector."""
    e = np.exp(s - s.max())
    return e / e.sum()


def _weighted_sum(p: np.ndarray, v_rows: np.ndarray) -> np.ndarray:
    """sum_t p_t v_t."""
    return p @ v_rows


# ---------------------------------------------------------------------------
# Cache write
# ---------------------------------------------------------------------------


def oracle_cache_write(k_pool: np.ndarray, v_pool: np.ndarray,
                       key: np.ndarray, value: np.ndarray,
                       slot_mapping: np.ndarray, block_size: int):
    """New tokens' K/V into their slots, as a bit copy.

    ``key``/``value`` are ``[N, n_kv_heads, d_head]``; token ``i`` goes to
    flat slot ``s = slot_mapping[i]`` = block ``s // block_size``, offset
    ``s % block_size``, for every KV head; ``s < 0`` skips the token.  The
    cache grows token by token into its blocks ("Serving", §23.4).  Returns new
    pools; the inputs are not modified."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for i, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        blk, off = s // block_size, s % block_size
        k_out[blk, :, off, :] = key[i]
        v_out[blk, :, off, :] = value[i]
    return k_out, v_out


# ---------------------------------------------------------------------------
# Block copy (copy-on-write)
# ---------------------------------------------------------------------------


def oracle_copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray,
                       block_pairs: np.ndarray):
    """Whole physical blocks duplicated in both pools, as a bit copy.

    Sequences that share a prefix share its blocks ("Serving", §23.4); with
    copy-on-write sharing (named in the "Paged Attention" summary on the
    inference-serving tag page) a shared block is duplicated before one
    sharer writes into it.  For each row ``(s, d)`` of ``block_pairs``, block
    ``d`` of each pool becomes a copy of block ``s`` as it was before the
    call (every KV head, position and dimension); a row naming a block
    outside the pool is skipped.  Returns new pools; the inputs are not
    modified."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    n_blocks = k_pool.shape[0]
    for s, d in np.asarray(block_pairs).reshape(-1, 2).tolist():
        if not (0 <= s < n_blocks and 0 <= d < n_blocks):
            continue
        k_out[d] = k_pool[s]
        v_out[d] = v_pool[s]
    return k_out, v_out


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------


def oracle_decode_row(q, k_pool, v_pool, block_table, context_lens, scale,
                      gqa_group, block_size, dtype, b, h, start=0, stop=None):
    """Attention output (fp64, ``[d_head]``) of query head ``h`` of sequence
    ``b`` over its cached positions ``start..stop-1`` (default: all of them).

    Also returns the row's logits so callers can form partition statistics.
    """
    n = int(context_lens[b])
    stop = n if stop is None else min(stop, n)
    kvh = _kv_head(h, gqa_group)
    k_rows = to_f64(_gather(k_pool, block_table[b], kvh, start, stop,
                            block_size), dtype)
    v_rows = to_f64(_gather(v_pool, block_table[b], kvh, start, stop,
                            block_size), dtype)
    q_h = to_f64(q[b, h], dtype)
    s = _logits(q_h, k_rows, float(np.float32(scale)))
    p = _softmax(s)
    return _weighted_sum(p, v_rows), s


def oracle_decode(q, k_pool, v_pool, block_table, context_lens, scale,
                  gqa_group, block_size, dtype, rows=None) -> np.ndarray:
    """Decode attention for every (sequence, query head), or only for the
    ``(b, h)`` pairs in ``rows``; fp64 ``[B, n_q_heads, d_head]`` (rows not
    asked for are NaN).  A sequence with ``context_len == 0`` gives a zero row
    (reading: the pages never produce one)."""
    B, Hq, D = q.shape
    out = np.full((B, Hq, D), np.nan)
    pairs = rows if rows is not None else [(b, h) for b in range(B)
                                           for h in range(Hq)]
    for b, h in pairs:
        if int(context_lens[b]) == 0:
            out[b, h] = 0.0
            continue
        out[b, h], _ = oracle_decode_row(q, k_pool, v_pool, block_table,
                                         context_lens, scale, gqa_group,
                                         block_size, dtype, b, h)
    return out


def oracle_decode_multi(q, k_pool, v_pool, block_table, context_lens, scale,
                        gqa_group, block_size, dtype, rows=None) -> np.ndarray:
    """Several query tokens per sequence, causal among themselves.

    The target model of speculative decoding checks all drafted tokens in one
    pass ("Serving", §23.5): ``q`` is ``[B, k, n_q_heads, d_head]``, the query
    of each sequence's last ``k`` positions, whose keys and values are
    already cached (``context_lens[b] = n`` counts them).  Token ``j`` sits
    at position ``n - k + j`` and, as in any causal decoder, attends to the
    positions up to and including its own: ``t < n - k + j + 1``.  A token
    that sees no position gives a zero row.  ``rows`` optionally lists
    ``(b, j, h)`` triples to compute (others are NaN).  Returns fp64
    ``[B, k, n_q_heads, d_head]``."""
    B, k, Hq, D = q.shape
    out = np.full((B, k, Hq, D), np.nan)
    trip = rows if rows is not None else [(b, j, h) for b in range(B)
                                          for j in range(k) for h in range(Hq)]
    for b, j, h in trip:
        visible = int(context_lens[b]) - k + j + 1
        if visible <= 0:
            out[b, j, h] = 0.0
            continue
        out[b, j, h], _ = oracle_decode_row(
            q[:, j], k_pool, v_pool, block_table, context_lens, scale,
            gqa_group, block_size, dtype, b, h, stop=visible)
    return out


# ---------------------------------------------------------------------------
# Split context: per-partition statistics and their merge
# ---------------------------------------------------------------------------


def oracle_partitions(q, k_pool, v_pool, block_table, context_lens, scale,
                      gqa_group, block_size, dtype, partition_size,
                      max_partitions=None, rows=None):
    """Per-partition softmax statistics.

    Partition ``p`` of sequence ``b`` covers positions
    ``[p*P, min((p+1)*P, ctx_b))``.  For each non-empty partition:

    * ``m[b,h,p]``  = max logit over the partition,
    * ``l[b,h,p]``  = sum_t exp(s_t - m),
    * ``o[b,h,p,:]`` = sum_t exp(s_t - m) v_t / l  (normalised).

    Empty partitions hold ``m = -inf, l = 0, o = 0``.  Returns fp64 arrays."""
    B, Hq, D = q.shape
    P = int(partition_size)
    if max_partitions is None:
        max_partitions = max(1, -(-int(np.max(context_lens)) // P))
    m = np.full((B, Hq, max_partitions), -np.inf)
    l = np.zeros((B, Hq, max_partitions))
    o = np.zeros((B, Hq, max_partitions, D))
    pairs = rows if rows is not None else [(b, h) for b in range(B)
                                           for h in range(Hq)]
    for b, h in pairs:
        n = int(context_lens[b])
        for p in range(-(-n // P)):
            o_p, s = oracle_decode_row(q, k_pool, v_pool, block_table,
                                       context_lens, scale, gqa_group,
                                       block_size, dtype, b, h,
                                       start=p * P, stop=(p + 1) * P)
            m[b, h, p] = s.max()
            l[b, h, p] = np.exp(s - s.max()).sum()
            o[b, h, p] = o_p
    return m, l, o


def oracle_merge(m, l, o, context_lens, partition_size) -> np.ndarray:
    """Combine per-partition statistics into the attention output.

    With ``M = max_p m_p`` and ``w_p = l_p exp(m_p - M)``:
    ``out = sum_p w_p o_p / sum_p w_p``.  This is the log-sum-exp identity:
    ``l_p exp(m_p)`` is the partition's softmax denominator and ``o_p`` its
    normalised numerator, so the weighted mean equals attention over the
    union of the partitions.  Sequences with no positions give zeros."""
    B, Hq, PM, D = o.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n_p = -(-int(context_lens[b]) // int(partition_size))
        if n_p == 0:
            continue
        for h in range(Hq):
            M = m[b, h, :n_p].max()
            w = l[b, h, :n_p] * np.exp(m[b, h, :n_p] - M)
            out[b, h] = (w[:, None] * o[b, h, :n_p]).sum(0) / w.sum()
    return out


# ---------------------------------------------------------------------------
# KV-cache size ("Serving", §23.1 The Memory Wall)
# ---------------------------------------------------------------------------


def kv_cache_bytes(n_layers: int, n_kv_heads: int, d_head: int, L: int,
                   B: int, n_bytes: int) -> int:
    """Bytes of the KV cache: 2 (keys and values) x layers x KV heads x head
    width x context length x batch x bytes per number."""
    return 2 * n_layers * n_kv_heads * d_head * L * B * n_bytes
