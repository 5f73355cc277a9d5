"""Seeded synthetic decode batches for the paged KV cache.

This module only *builds inputs*: context lengths, the physical placement of
blocks, per-sequence block tables, the slot of each sequence's new token, and
random q/K/V values rounded to the storage dtype.  It holds none of the
attention arithmetic, so the fp64 oracle and the HIP path can both be fed from
it without sharing any of the method's code.

Layout of what it returns (all row-major, numpy):

* ``q``            ``[B, n_q_heads, d_head]``              storage dtype
* ``k_pool``/``v_pool`` ``[n_blocks, n_kv_heads, block_size, d_head]``
  storage dtype.  A block of ``block_size`` consecutive token positions of one
  sequence lives in one physical block ("Serving", §23.4 Paged Attention: the
  cache is kept in small fixed-size blocks of, say, 16 tokens, with a
  per-sequence table from positions to blocks).
* ``block_table``  ``[B, max_blocks]`` int32, -1 beyond each sequence's blocks
* ``context_lens`` ``[B]`` int32; position ``ctx-1`` is the token decoded this
  step and is *not* in the pool until the cache write puts it there
* ``key_new``/``value_new`` ``[B, n_kv_heads, d_head]`` storage dtype
* ``slot_mapping`` ``[B]`` int32, flat slot ``phys_block * block_size + offset``

Storage dtypes: ``f32`` -> ``np.float32``, ``f16`` -> ``np.float16``,
``bf16`` -> ``np.uint16`` holding bfloat16 bit patterns (numpy has no bf16).

Pool slots that hold no token (the tail of each sequence's last block, unused
blocks, and the new token's slot before it is written) are filled with NaN
when ``poison=True`` so that a kernel which reads them without masking is
caught.  Randomness: ``numpy.random.SeedSequence(seed).spawn(6)`` gives one
``Generator(PCG64DXSM)`` each for the lengths, q, K, V, the new tokens' K then
V, and the block placement, so re-blocking a config keeps every token's
values.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Callable, Dict, Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


# --------------------------------------------------------------------------
# Encoding fp32 draws into the storage dtypes
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns.  NaN maps to the quiet NaN 0x7FC0."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values -> storage array of ``dtype`` (RNE rounding)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def nan_value(dtype: str):
    """The NaN poison value in storage form."""
    if dtype == "bf16":
        return np.uint16(0x7FC0)
    return STORAGE[dtype](np.nan)


# --------------------------------------------------------------------------
# Config registry
# --------------------------------------------------------------------------

LengthFn = Callable[[np.random.Generator, int], np.ndarray]


@dataclasses.dataclass(frozen=True)
class Config:
    """One decode step of one layer, shaped like the pages' workloads."""

    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    d_head: int
    block_size: int
    dtype: str
    max_context: int            # upper bound of the length distribution
    lengths: LengthFn           # (rng, batch) -> int array of context lengths
    std: float = 1.0
    pool_blocks: Optional[int] = None   # None: exactly the blocks in use
    prefix_len: int = 0         # tokens shared by every sequence (block aligned)
    partition_size: int = 512
    description: str = ""

    @property
    def gqa_group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_blocks(self) -> int:
        return -(-self.max_context // self.block_size)

    @property
    def max_partitions(self) -> int:
        return -(-self.max_context // self.partition_size)

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d_head)))

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def _fixed(values):
    arr = np.asarray(values, dtype=np.int64)

    def fn(rng, b):
        assert b == len(arr), "fixed lengths need batch == len(values)"
        return arr.copy()
    return fn


def _uniform(lo, hi):
    def fn(rng, b):
        return rng.integers(lo, hi, size=b, endpoint=True)
    return fn


def _constant(n):
    def fn(rng, b):
        return np.full(b, n, dtype=np.int64)
    return fn


def _lognormal(median, sigma, lo, hi):
    def fn(rng, b):
        z = rng.normal(math.log(median), sigma, size=b)
        return np.clip(np.rint(np.exp(z)), lo, hi).astype(np.int64)
    return fn


def _prefix_plus_uniform(prefix, lo, hi):
    def fn(rng, b):
        return prefix + rng.integers(lo, hi, size=b, endpoint=True)
    return fn


CONFIGS: Dict[str, Config] = {
    "tiny": Config(
        name="tiny", batch=4, n_q_heads=4, n_kv_heads=2, d_head=64,
        block_size=16, dtype="f32", max_context=100,
        lengths=_fixed([17, 48, 63, 100]), pool_blocks=32,
        description="1 layer, B=4, 4/2 heads, d64, bs16, fp32, "
                    "ctx {17,48,63,100}, 32-block pool"),
    "qwen2.5-1.5b": Config(
        name="qwen2.5-1.5b", batch=64, n_q_heads=12, n_kv_heads=2, d_head=128,
        block_size=16, dtype="bf16", max_context=4096,
        lengths=_uniform(128, 4096), pool_blocks=20000,
        # not fixed by the workload: among 256..2048 on MI355X, 1536 is the
        # fastest (attention 33.6-33.8 us; 34.0-34.3 at 640, 35.5-35.7 at 768)
        partition_size=1536,
        description="12/2 heads, d128, bf16, B=64, ctx U[128,4096], "
                    "20k-block pool, 1536-token partitions"),
    "llama2-7b": Config(
        name="llama2-7b", batch=32, n_q_heads=32, n_kv_heads=32, d_head=128,
        block_size=16, dtype="f16", max_context=4096,
        lengths=_constant(4096), std=0.5,
        # not fixed by the workload: one partition per sequence is the
        # fastest (fused step 329.7/332.2/337.6 us at 4096/2048/1024); the
        # partitioned step, 327.0-329.3 us, is within ~1.5 % of the fused
        # step and the single pass (329.8-334.4 us) on two MI355X boxes
        partition_size=4096,
        description="MHA 32/32 heads, d128, fp16, B=32, ctx 4096, "
                    "pool exactly B*L/16 blocks, values N(0, 0.5), "
                    "4096-token partitions"),
    "llama3-8b": Config(
        name="llama3-8b", batch=128, n_q_heads=32, n_kv_heads=8, d_head=128,
        block_size=16, dtype="bf16", max_context=8192,
        lengths=_lognormal(1024, 1.0, 16, 8192),
        # not fixed by the workload: the fastest of 2048..4096 on MI355X
        # (step 148.8/152.5/146.7/147.8/149.6 us at 2048/2560/3072/3584/4096)
        partition_size=3072,
        description="GQA 32/8 heads, d128, bf16, B=128, ctx log-normal "
                    "(median 1024, sigma 1) clipped to [16, 8192], "
                    "3072-token partitions"),
    "shared-prefix": Config(
        name="shared-prefix", batch=256, n_q_heads=32, n_kv_heads=8,
        d_head=128, block_size=16, dtype="bf16", max_context=2048 + 6144,
        lengths=_prefix_plus_uniform(2048, 1, 6144), prefix_len=2048,
        partition_size=512,
        description="GQA 32/8 heads, d128, bf16, B=256, 2048-token shared "
                    "prefix + private suffix U[1,6144], 512-token partitions"),
}

# The decode batch the throughput figure is quoted on.
HEADLINE = "llama3-8b"


# --------------------------------------------------------------------------
# The generated batch
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    cfg: Config
    seed: int
    context_lens: np.ndarray    # [B] int32
    block_table: np.ndarray     # [B, max_blocks] int32
    q: np.ndarray               # [B, Hq, D]
    k_pool: np.ndarray          # [n_blocks, Hkv, BS, D], before the write
    v_pool: np.ndarray
    key_new: np.ndarray         # [B, Hkv, D]
    value_new: np.ndarray
    slot_mapping: np.ndarray    # [B] int32

    @property
    def n_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def scale(self) -> float:
        return self.cfg.scale

    # --- byte accounting (algorithmic, not measured) ----------------------
    def kv_bytes_logical(self) -> int:
        """K and V bytes a decode step reads: every cached position of every
        sequence, for every KV head, counted once per sequence."""
        c = self.cfg
        return int(self.context_lens.astype(np.int64).sum()) * c.n_kv_heads * \
            c.d_head * 2 * DTYPE_BYTES[c.dtype]

    def kv_bytes_unique(self) -> int:
        """Bytes of the distinct (block, kv-head) tiles a step touches; differs
        from the logical figure only where blocks are shared."""
        c = self.cfg
        tok = 0
        seen = set()
        for b in range(c.batch):
            n = int(self.context_lens[b])
            nblk = -(-n // c.block_size)
            for j in range(nblk):
                p = int(self.block_table[b, j])
                used = min(c.block_size, n - j * c.block_size)
                if p in seen:
                    continue
                seen.add(p)
                tok += used
        return tok * c.n_kv_heads * c.d_head * 2 * DTYPE_BYTES[c.dtype]


_CHUNK = 1 << 22   # values per chunk of the K/V draws


def _streams(seed: int):
    """Independent generators for lengths, q, K, V, the new tokens' K/V and
    block placement, spawned from one seed."""
    kids = np.random.SeedSequence(seed).spawn(6)
    return [np.random.Generator(np.random.PCG64DXSM(k)) for k in kids]


def _fill_tokens(rng, pool, blk, off, std, dtype) -> None:
    """Draw ``len(blk)`` tokens' values (float32 normals times ``std``,
    rounded to ``dtype``) and store token i at ``pool[blk[i], :, off[i], :]``.
    Works in chunks so no pool-sized temporaries are made."""
    _, H, _, D = pool.shape
    per = H * D
    step = max(1, _CHUNK // per)
    buf = np.empty(step * per, dtype=np.float32)
    for s in range(0, len(blk), step):
        n = min(step, len(blk) - s)
        x = buf[:n * per]
        rng.standard_normal(out=x, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        pool[blk[s:s + n], :, off[s:s + n], :] = encode(x, dtype).reshape(n, H, D)


def _draw_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    ctx = np.asarray(cfg.lengths(rng, cfg.batch), dtype=np.int64)
    return np.minimum(ctx, cfg.max_context)


def draw_lengths(cfg: Config | str, seed: int = 0) -> np.ndarray:
    """The context lengths ``make_workload(cfg, seed)`` would produce, without
    drawing any values."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    return _draw_lengths(cfg, _streams(seed)[0]).astype(np.int32)


def make_workload(cfg: Config | str, seed: int = 0, *, poison: bool = True,
                  batch: Optional[int] = None,
                  max_context: Optional[int] = None,
                  block_size: Optional[int] = None) -> Workload:
    """Build the seeded batch for ``cfg``.

    ``batch``/``max_context``/``block_size`` shrink or re-block a config while
    keeping its distributions (lengths are clipped to ``max_context``)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if batch is not None:
        cfg = cfg.with_(batch=batch)
    if block_size is not None:
        cfg = cfg.with_(block_size=block_size)
    if max_context is not None:
        cfg = cfg.with_(max_context=max_context)
    rl, rq, rk, rv, rn, rp = _streams(seed)
    B, Hq, Hkv, D, BS = (cfg.batch, cfg.n_q_heads, cfg.n_kv_heads,
                          cfg.d_head, cfg.block_size)
    assert Hq % Hkv == 0
    assert cfg.prefix_len % BS == 0

    # 1. lengths
    ctx = _draw_lengths(cfg, rl)
    assert (ctx >= 1).all()
    if cfg.prefix_len:
        assert (ctx > cfg.prefix_len).all()

    # 2. values: q and the new tokens' K/V here; K and V of the distinct
    #    cached tokens (prefix tokens once, then each sequence's own tokens
    #    before its new one, in that order) are drawn in chunks straight into
    #    the pool in step 4.
    q = encode(rq.standard_normal((B, Hq, D), dtype=np.float32) * cfg.std,
               cfg.dtype)
    n_tok = cfg.prefix_len + int((ctx - 1 - cfg.prefix_len).sum())
    key_new = encode(rn.standard_normal((B, Hkv, D), dtype=np.float32)
                     * cfg.std, cfg.dtype)
    value_new = encode(rn.standard_normal((B, Hkv, D), dtype=np.float32)
                       * cfg.std, cfg.dtype)

    # 3. placement: logical blocks in canonical order (the shared prefix
    #    blocks first, then each sequence's private blocks) take the first
    #    ids of a random permutation of the pool.
    n_prefix_blocks = cfg.prefix_len // BS
    nblk = -(-ctx // BS)
    n_private = int((nblk - n_prefix_blocks).sum())
    n_used = n_prefix_blocks + n_private
    n_blocks = cfg.pool_blocks if cfg.pool_blocks is not None else n_used
    assert n_blocks >= n_used, "pool too small"
    phys = rp.permutation(n_blocks)[:n_used].astype(np.int64)
    MB = cfg.max_blocks
    table = np.full((B, MB), -1, dtype=np.int32)
    cursor = n_prefix_blocks
    for b in range(B):
        table[b, :n_prefix_blocks] = phys[:n_prefix_blocks]
        k = int(nblk[b]) - n_prefix_blocks
        table[b, n_prefix_blocks:n_prefix_blocks + k] = phys[cursor:cursor + k]
        cursor += k

    # 4. lay the drawn tokens into the pool through the tables
    st = STORAGE[cfg.dtype]
    fill = nan_value(cfg.dtype) if poison else st(0)
    k_pool = np.full((n_blocks, Hkv, BS, D), fill, dtype=st)
    v_pool = np.full((n_blocks, Hkv, BS, D), fill, dtype=st)
    tok_b = np.empty(n_tok, dtype=np.int64)
    tok_t = np.empty(n_tok, dtype=np.int64)
    tok_b[:cfg.prefix_len] = 0
    tok_t[:cfg.prefix_len] = np.arange(cfg.prefix_len)
    cur = cfg.prefix_len
    for b in range(B):
        n = int(ctx[b]) - 1 - cfg.prefix_len
        tok_b[cur:cur + n] = b
        tok_t[cur:cur + n] = np.arange(cfg.prefix_len, cfg.prefix_len + n)
        cur += n
    blk = table[tok_b, tok_t // BS].astype(np.int64)
    off = tok_t % BS
    del tok_b, tok_t
    _fill_tokens(rk, k_pool, blk, off, cfg.std, cfg.dtype)
    _fill_tokens(rv, v_pool, blk, off, cfg.std, cfg.dtype)
    del blk, off

    pos = ctx - 1
    slot = table[np.arange(B), pos // BS].astype(np.int64) * BS + pos % BS
    return Workload(cfg=cfg, seed=seed,
                    context_lens=ctx.astype(np.int32),
                    block_table=table, q=q, k_pool=k_pool, v_pool=v_pool,
                    key_new=key_new, value_new=value_new,
                    slot_mapping=slot.astype(np.int32))


def make_custom(context_lens, *, n_q_heads: int, n_kv_heads: int, d_head: int,
                block_size: int, dtype: str, seed: int = 0, std: float = 1.0,
                pool_blocks: Optional[int] = None, prefix_len: int = 0,
                max_context: Optional[int] = None, partition_size: int = 512,
                poison: bool = True) -> Workload:
    """A batch with explicit context lengths (edge cases, small parity runs)."""
    ctx = [int(c) for c in context_lens]
    cfg = Config(name="custom", batch=len(ctx), n_q_heads=n_q_heads,
                 n_kv_heads=n_kv_heads, d_head=d_head, block_size=block_size,
                 dtype=dtype, max_context=max_context or max(ctx + [1]),
                 lengths=_fixed(ctx), std=std, pool_blocks=pool_blocks,
                 prefix_len=prefix_len, partition_size=partition_size)
    return make_workload(cfg, seed, poison=poison)


def make_copy_pairs(n_blocks: int, n_pairs: int, seed: int = 0, *,
                    invalid: int = 0) -> np.ndarray:
    """[n_pairs + invalid, 2] int32 (source, destination) rows for a block
    copy over a pool of n_blocks: distinct destinations, none of them a
    source; ``invalid`` extra rows name a block outside the pool."""
    if 2 * n_pairs > n_blocks:
        raise ValueError("need 2 * n_pairs <= n_blocks")
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(7)[6])
    perm = rng.permutation(n_blocks)
    dst = perm[:n_pairs]
    src = rng.choice(perm[n_pairs:], size=n_pairs, replace=True)
    pairs = np.stack([src, dst], axis=1).astype(np.int32)
    if invalid:
        bad = np.stack([rng.choice([-1, n_blocks], invalid),
                        rng.integers(0, n_blocks, invalid)], axis=1)
        bad[1::2] = bad[1::2, ::-1]          # half with a bad destination
        pairs = np.concatenate([pairs, bad.astype(np.int32)])
        pairs = pairs[rng.permutation(len(pairs))]
    return np.ascontiguousarray(pairs, dtype=np.int32)


def make_multi_queries(w: Workload, n_queries: int, seed: int = 0) -> np.ndarray:
    """[B, n_queries, n_q_heads, d_head] queries for the last n_queries
    positions of each sequence (float32 normals times the batch's std,
    rounded to its dtype), from a stream of their own."""
    c = w.cfg
    rng = np.random.Generator(np.random.PCG64DXSM(
        np.random.SeedSequence(seed).spawn(8)[7]))
    x = rng.standard_normal((c.batch, n_queries, c.n_q_heads, c.d_head),
                            dtype=np.float32)
    if c.std != 1.0:
        x *= np.float32(c.std)
    return encode(x, c.dtype)


def multi_token_slots(w: Workload, n_queries: int) -> np.ndarray:
    """[B * n_queries] int32 flat slots of each sequence's last n_queries
    positions (the tokens a verify pass writes; -1 below position 0)."""
    c = w.cfg
    out = np.full((c.batch, n_queries), -1, dtype=np.int64)
    for b in range(c.batch):
        n = int(w.context_lens[b])
        for j in range(n_queries):
            pos = n - n_queries + j
            if pos >= 0:
                out[b, j] = int(w.block_table[b, pos // c.block_size]) * \
                    c.block_size + pos % c.block_size
    return out.reshape(-1).astype(np.int32)


# The "Serving" §23.4 widget: a 96-block pool of 16-token blocks and eight
# requests arriving over time.  The page gives no sizes; these are chosen so
# that its two statements can be checked: a worst case of 384 tokens (24
# blocks, so four reservations fill the pool) and final lengths of at most
# 192 tokens (12 blocks, so eight paged requests fit together).
WIDGET = dict(n_blocks=96, block_size=16, n_requests=8, max_len=384,
              arrival_gap=8, prompt=(16, 64), final=(96, 192))


def widget_requests(seed: int = 0):
    """(arrivals, prompt_lens, final_lens) of the widget's eight requests."""
    w = WIDGET
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(9)[8])
    n = w["n_requests"]
    arrivals = [i * w["arrival_gap"] for i in range(n)]
    prompts = [int(x) for x in rng.integers(w["prompt"][0], w["prompt"][1] + 1, n)]
    finals = [int(x) for x in rng.integers(w["final"][0], w["final"][1] + 1, n)]
    return arrivals, prompts, finals
