"""Pins for the fp64 oracle: checks against things other than the oracle.

Each pin ties a part of the oracle to something independent of it: values the
pages print, a library routine (torch's CPU scaled-dot-product attention), a
closed form, or an invariant the paged layout must satisfy.  The mutation
tests at the end swap one internal step of the oracle for a plausible mistake
and assert that at least one pin then fails.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import paged_attention as pa_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers: build a paged pool from contiguous per-sequence K/V (test-side)
# ---------------------------------------------------------------------------

def _draw(rng, ctx, Hq, Hkv, D, qscale=1.0):
    """Random queries and contiguous per-sequence K/V ``[Hkv, n, D]``."""
    q = rng.standard_normal((len(ctx), Hq, D)) * qscale
    seqs = [(rng.standard_normal((Hkv, n, D)), rng.standard_normal((Hkv, n, D)))
            for n in ctx]
    return q, seqs


def _page(rng, seqs, BS, extra_blocks=3):
    """Scatter contiguous K/V into a randomly permuted pool of BS-token
    blocks; unused slots hold NaN.  Returns (pool_k, pool_v, table, ctx)."""
    ctx = [K.shape[1] for K, _ in seqs]
    Hkv, D = seqs[0][0].shape[0], seqs[0][0].shape[2]
    nblk = [-(-n // BS) for n in ctx]
    n_blocks = sum(nblk) + extra_blocks
    perm = rng.permutation(n_blocks)
    table = np.full((len(ctx), max(nblk + [1])), -1, dtype=np.int32)
    pool_k = np.full((n_blocks, Hkv, BS, D), np.nan)
    pool_v = np.full((n_blocks, Hkv, BS, D), np.nan)
    cur = 0
    for b, (K, V) in enumerate(seqs):
        for j in range(nblk[b]):
            table[b, j] = perm[cur]
            cur += 1
        for t in range(ctx[b]):
            blk = table[b, t // BS]
            pool_k[blk, :, t % BS, :] = K[:, t, :]
            pool_v[blk, :, t % BS, :] = V[:, t, :]
    return pool_k, pool_v, table, np.asarray(ctx, dtype=np.int32)


def _contiguous_case(rng, ctx, Hq, Hkv, D, BS, extra_blocks=3, qscale=1.0):
    """Queries, a paged pool holding contiguous per-sequence K/V, and that
    contiguous data: (q, pool_k, pool_v, table, ctx, [(K_b, V_b)])."""
    q, seqs = _draw(rng, ctx, Hq, Hkv, D, qscale)
    pk, pv, table, cl = _page(rng, seqs, BS, extra_blocks)
    return q, pk, pv, table, cl, seqs


def _sdpa_reference(q, seqs, scale, G):
    """torch CPU fp64 scaled_dot_product_attention on the contiguous data."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for b, (K, V) in enumerate(seqs):
        qt = torch.from_numpy(q[b][None, :, None, :])            # [1,Hq,1,D]
        Kt = torch.from_numpy(np.repeat(K, G, axis=0)[None])     # [1,Hq,n,D]
        Vt = torch.from_numpy(np.repeat(V, G, axis=0)[None])
        o = F.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
        out[b] = o[0, :, 0, :].numpy()
    return out


CASES = [
    # (ctx list, Hq, Hkv, D, BS)
    ([1, 5, 16, 17, 40], 4, 2, 8, 4),
    ([3, 33, 64], 6, 2, 16, 16),
    ([100, 7], 8, 8, 4, 8),
    ([31, 32, 1], 3, 1, 8, 32),
    ([50], 12, 4, 8, 2),
]


@pytest.mark.parametrize("ctx,Hq,Hkv,D,BS", CASES)
def test_paged_equals_contiguous_sdpa(ctx, Hq, Hkv, D, BS):
    """Pin (library routine): the paged oracle equals torch's fp64 SDPA run
    on the same K/V stored contiguously, with KV heads repeated per group."""
    rng = np.random.default_rng(1234 + Hq * 7 + BS)
    q, pk, pv, table, cl, seqs = _contiguous_case(rng, ctx, Hq, Hkv, D, BS)
    scale = 1.0 / math.sqrt(D)
    got = oracle.oracle_decode(q, pk, pv, table, cl, scale, Hq // Hkv, BS,
                               "f32")
    ref = _sdpa_reference(q, seqs, float(np.float32(scale)), Hq // Hkv)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def _sdpa_multi_reference(q, seqs, scale, G):
    """torch CPU fp64 SDPA for k query tokens per sequence with an explicit
    mask: token j (position n - k + j) may attend to keys t <= n - k + j."""
    B, k, Hq, D = q.shape
    out = np.zeros((B, k, Hq, D))
    for b, (K, V) in enumerate(seqs):
        n = K.shape[1]
        qt = torch.from_numpy(np.ascontiguousarray(q[b].transpose(1, 0, 2))[None])
        Kt = torch.from_numpy(np.repeat(K, G, axis=0)[None])     # [1,Hq,n,D]
        Vt = torch.from_numpy(np.repeat(V, G, axis=0)[None])
        j = torch.arange(k)[:, None]
        t = torch.arange(n)[None, :]
        mask = t <= (n - k + j)                                   # [k, n]
        o = F.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask,
                                           scale=scale)
        out[b] = o[0].numpy().transpose(1, 0, 2)
    return out


@pytest.mark.parametrize("ctx,Hq,Hkv,D,BS,k", [
    ([5, 17, 40], 4, 2, 8, 4, 4), ([33, 64, 4], 8, 2, 16, 16, 4),
    ([100, 7], 4, 4, 8, 8, 3), ([31, 2], 6, 2, 8, 32, 2)])
def test_multi_query_equals_masked_sdpa(ctx, Hq, Hkv, D, BS, k):
    """Pin (library routine): k causal query tokens per sequence equal
    torch's fp64 SDPA with the bottom-right causal mask."""
    rng = np.random.default_rng(sum(ctx) + k)
    q, pk, pv, table, cl, seqs = _contiguous_case(rng, ctx, Hq, Hkv, D, BS)
    qm = rng.standard_normal((len(ctx), k, Hq, D))
    scale = 1.0 / math.sqrt(D)
    got = oracle.oracle_decode_multi(qm, pk, pv, table, cl, scale, Hq // Hkv,
                                     BS, "f32")
    ref = _sdpa_multi_reference(qm, seqs, float(np.float32(scale)), Hq // Hkv)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_multi_query_single_token_is_decode():
    """Special case: one query token is single-token decode."""
    rng = np.random.default_rng(61)
    q, pk, pv, table, cl, _ = _contiguous_case(rng, [9, 30], 4, 2, 8, 8)
    got = oracle.oracle_decode_multi(q[:, None], pk, pv, table, cl, 0.3, 2, 8,
                                     "f32")
    want = oracle.oracle_decode(q, pk, pv, table, cl, 0.3, 2, 8, "f32")
    assert np.array_equal(got[:, 0], want)


def test_multi_query_token_without_positions_is_zero():
    """A sequence shorter than k: its first tokens see nothing (zero rows),
    the rest see a causal prefix."""
    rng = np.random.default_rng(67)
    q, pk, pv, table, cl, seqs = _contiguous_case(rng, [2], 2, 1, 4, 4)
    qm = rng.standard_normal((1, 4, 2, 4))
    got = oracle.oracle_decode_multi(qm, pk, pv, table, cl, 0.5, 2, 4, "f32")
    assert (got[0, :2] == 0).all()
    V = seqs[0][1][0]
    np.testing.assert_allclose(got[0, 2, 0], V[0], rtol=0, atol=1e-15)


def test_stress_large_logits_equal_sdpa():
    """Pin: logits of magnitude ~100s (q scaled up) still match SDPA, which
    needs the max subtraction in the softmax."""
    rng = np.random.default_rng(7)
    q, pk, pv, table, cl, seqs = _contiguous_case(rng, [20, 45], 4, 2, 8, 8,
                                                  qscale=300.0)
    scale = 1.0 / math.sqrt(8)
    got = oracle.oracle_decode(q, pk, pv, table, cl, scale, 2, 8, "f32")
    ref = _sdpa_reference(q, seqs, float(np.float32(scale)), 2)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-9)


def test_permutation_invariance():
    """Invariant: relabelling physical blocks (pool rows and table entries by
    the same permutation) leaves every output bit-identical."""
    rng = np.random.default_rng(3)
    q, pk, pv, table, cl, _ = _contiguous_case(rng, [9, 30, 47], 4, 2, 8, 8)
    n_blocks = pk.shape[0]
    pi = rng.permutation(n_blocks)          # new id of old block i
    pk2 = np.empty_like(pk)
    pv2 = np.empty_like(pv)
    pk2[pi] = pk
    pv2[pi] = pv
    table2 = np.where(table >= 0, pi[np.maximum(table, 0)], -1).astype(np.int32)
    a = oracle.oracle_decode(q, pk, pv, table, cl, 0.3, 2, 8, "f32")
    b = oracle.oracle_decode(q, pk2, pv2, table2, cl, 0.3, 2, 8, "f32")
    assert np.array_equal(a, b)


def test_block_size_layouts_agree():
    """Invariant: the same logical content stored with 4-, 8- and 16-token
    blocks gives the same outputs."""
    rng = np.random.default_rng(11)
    q, seqs = _draw(rng, [5, 16, 37], 4, 2, 8)
    outs = []
    for BS in (4, 8, 16):
        pk, pv, table, cl = _page(rng, seqs, BS)
        outs.append(oracle.oracle_decode(q, pk, pv, table, cl, 0.25, 2, BS,
                                         "f32"))
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=0, atol=1e-13)


def test_softmax_weights_sum_to_one():
    """Closed form: with every V row equal to 1 the output is the sum of the
    softmax weights, which is 1."""
    rng = np.random.default_rng(5)
    q, pk, pv, table, cl, _ = _contiguous_case(rng, [1, 13, 64], 6, 3, 8, 4)
    pv = np.where(np.isnan(pv), np.nan, 1.0)
    out = oracle.oracle_decode(q, pk, pv, table, cl, 0.7, 2, 4, "f32")
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-12)


def test_single_position_returns_its_value():
    """Closed form: one cached position gets weight 1, so out = v_0."""
    rng = np.random.default_rng(6)
    q, pk, pv, table, cl, seqs = _contiguous_case(rng, [1, 1], 4, 2, 8, 16)
    out = oracle.oracle_decode(q, pk, pv, table, cl, 0.5, 2, 16, "f32")
    for b in range(2):
        V = seqs[b][1]
        for h in range(4):
            assert np.array_equal(out[b, h], V[h // 2, 0])


def test_zero_query_and_constant_keys_average_values():
    """Closed form: q = 0, or all keys equal, makes every logit equal, so the
    output is the plain mean of the value rows."""
    rng = np.random.default_rng(8)
    q, pk, pv, table, cl, seqs = _contiguous_case(rng, [7, 20], 4, 2, 8, 4)
    out0 = oracle.oracle_decode(np.zeros_like(q), pk, pv, table, cl, 0.5, 2, 4,
                                "f32")
    pk_const = np.where(np.isnan(pk), np.nan, 0.0) + 0.3
    out1 = oracle.oracle_decode(q, pk_const, pv, table, cl, 0.5, 2, 4, "f32")
    for b in range(2):
        mean = seqs[b][1].mean(axis=1)          # [Hkv, D]
        for h in range(4):
            np.testing.assert_allclose(out0[b, h], mean[h // 2], atol=1e-13)
            np.testing.assert_allclose(out1[b, h], mean[h // 2], atol=1e-13)


def test_two_position_worked_example():
    """Closed form: logits 0 and ln 3 give weights 1/4 and 3/4."""
    D = 4
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = 1.0
    pk = np.zeros((2, 1, 1, D))           # block size 1, blocks swapped
    pv = np.zeros((2, 1, 1, D))
    pk[1, 0, 0, 0] = 0.0                  # position 0 -> block 1
    pk[0, 0, 0, 0] = math.log(3.0)        # position 1 -> block 0
    pv[1, 0, 0] = [4.0, 0.0, 8.0, -4.0]
    pv[0, 0, 0] = [0.0, 4.0, 0.0, 4.0]
    table = np.array([[1, 0]], dtype=np.int32)
    out = oracle.oracle_decode(q, pk, pv, table, np.array([2]), 1.0, 1, 1,
                               "f32")
    np.testing.assert_allclose(out[0, 0], [1.0, 3.0, 2.0, 2.0], atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv_heads():
    """Special case: G > 1 equals G = 1 after repeating each KV head G times
    in the pool (MHA is the G = 1 case)."""
    rng = np.random.default_rng(21)
    G = 3
    q, pk, pv, table, cl, _ = _contiguous_case(rng, [11, 29], 6, 2, 8, 8)
    gqa = oracle.oracle_decode(q, pk, pv, table, cl, 0.4, G, 8, "f32")
    mha = oracle.oracle_decode(q, np.repeat(pk, G, axis=1),
                               np.repeat(pv, G, axis=1), table, cl, 0.4, 1, 8,
                               "f32")
    np.testing.assert_allclose(gqa, mha, rtol=0, atol=1e-14)


def test_shared_prefix_rows_identical():
    """Invariant: sequences whose tables share the same prefix blocks and the
    same suffix contents, with equal queries, give equal outputs."""
    rng = np.random.default_rng(31)
    BS, Hkv, D = 4, 2, 8
    n_blocks = 12
    pk = rng.standard_normal((n_blocks, Hkv, BS, D))
    pv = rng.standard_normal((n_blocks, Hkv, BS, D))
    pk[9] = pk[5]
    pv[9] = pv[5]                          # block 9 is a copy of block 5
    table = np.array([[2, 7, 5], [2, 7, 9]], dtype=np.int32)
    q = np.repeat(rng.standard_normal((1, 4, D)), 2, axis=0)
    out = oracle.oracle_decode(q, pk, pv, table, np.array([10, 10]), 0.3, 2,
                               BS, "f32")
    assert np.array_equal(out[0], out[1])


@pytest.mark.parametrize("P", [4, 8, 12, 512])
def test_partition_merge_equals_unsplit(P):
    """Closed form (log-sum-exp identity): merging per-partition statistics
    gives the unsplit attention for any block-aligned partition size."""
    rng = np.random.default_rng(41)
    q, pk, pv, table, cl, _ = _contiguous_case(rng, [1, 4, 13, 50], 4, 2, 8, 4)
    full = oracle.oracle_decode(q, pk, pv, table, cl, 0.5, 2, 4, "f32")
    m, l, o = oracle.oracle_partitions(q, pk, pv, table, cl, 0.5, 2, 4, "f32",
                                       P)
    merged = oracle.oracle_merge(m, l, o, cl, P)
    np.testing.assert_allclose(merged, full, rtol=0, atol=1e-13)


def test_single_partition_is_identity():
    """Closed form: with one partition covering everything, the normalised
    partial output is the answer and l is the softmax denominator."""
    rng = np.random.default_rng(43)
    q, pk, pv, table, cl, seqs = _contiguous_case(rng, [9, 24], 4, 2, 8, 8)
    full = oracle.oracle_decode(q, pk, pv, table, cl, 0.5, 2, 8, "f32")
    m, l, o = oracle.oracle_partitions(q, pk, pv, table, cl, 0.5, 2, 8, "f32",
                                       64)
    np.testing.assert_allclose(o[:, :, 0, :], full, atol=1e-14)
    for b in range(2):
        K = seqs[b][0]
        for h in range(4):
            s = 0.5 * (K[h // 2] @ q[b, h])
            assert m[b, h, 0] == pytest.approx(s.max(), abs=1e-14)
            assert l[b, h, 0] == pytest.approx(np.exp(s - s.max()).sum(),
                                               rel=1e-13)


def test_zero_context_gives_zeros():
    """Reading (pages silent): an empty sequence decodes to a zero row, and
    has no partitions."""
    rng = np.random.default_rng(47)
    q, pk, pv, table, cl, _ = _contiguous_case(rng, [5, 6], 4, 2, 8, 4)
    cl = np.array([0, 6], dtype=np.int32)
    out = oracle.oracle_decode(q, pk, pv, table, cl, 0.5, 2, 4, "f32")
    assert np.array_equal(out[0], np.zeros((4, 8)))
    m, l, o = oracle.oracle_partitions(q, pk, pv, table, cl, 0.5, 2, 4, "f32",
                                       4)
    merged = oracle.oracle_merge(m, l, o, cl, 4)
    assert np.array_equal(merged[0], np.zeros((4, 8)))
    assert np.isneginf(m[0]).all() and (l[0] == 0).all()


# ---------------------------------------------------------------------------
# cache write
# ---------------------------------------------------------------------------

def _flat_slot_view(pool):
    """[n_blocks, Hkv, BS, D] -> [n_blocks*BS, Hkv, D]: slot-major copy."""
    nb, H, BS, D = pool.shape
    return pool.transpose(0, 2, 1, 3).reshape(nb * BS, H, D)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_cache_write_matches_flat_slot_view(dtype):
    """Pin: after the write, reading the pool as a slot-major array at index
    ``slot`` returns the token bit for bit; every other slot is unchanged."""
    rng = np.random.default_rng(51)
    nb, H, BS, D = 10, 3, 8, 16
    st = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    if dtype == "bf16":
        pool_k = rng.integers(0, 2**16, (nb, H, BS, D)).astype(np.uint16)
        pool_v = rng.integers(0, 2**16, (nb, H, BS, D)).astype(np.uint16)
        key = rng.integers(0, 2**16, (6, H, D)).astype(np.uint16)
        val = rng.integers(0, 2**16, (6, H, D)).astype(np.uint16)
    else:
        pool_k = rng.standard_normal((nb, H, BS, D)).astype(st)
        pool_v = rng.standard_normal((nb, H, BS, D)).astype(st)
        key = rng.standard_normal((6, H, D)).astype(st)
        val = rng.standard_normal((6, H, D)).astype(st)
    slots = np.array([0, 79, -1, 17, 40, 8], dtype=np.int32)
    k2, v2 = oracle.oracle_cache_write(pool_k, pool_v, key, val, slots, BS)
    fk, fv = _flat_slot_view(k2), _flat_slot_view(v2)
    fk0, fv0 = _flat_slot_view(pool_k), _flat_slot_view(pool_v)
    written = set()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        written.add(int(s))
        assert fk[s].tobytes() == key[i].tobytes()
        assert fv[s].tobytes() == val[i].tobytes()
    for s in range(nb * BS):
        if s not in written:
            assert fk[s].tobytes() == fk0[s].tobytes()
            assert fv[s].tobytes() == fv0[s].tobytes()
    # the inputs are untouched
    assert not np.shares_memory(k2, pool_k)


def _coded_pools(nb, H, BS, D):
    """f32 pools whose element (b, h, p, d) stores its own index code
    ((b*H + h)*BS + p)*D + d in K and -1 - code in V (exact integers)."""
    code = np.arange(nb * H * BS * D, dtype=np.float64).reshape(nb, H, BS, D)
    return code.astype(np.float32), (-1.0 - code).astype(np.float32)


def test_copy_blocks_moves_whole_blocks():
    """Pin: decoding the stored codes after the copy, every element of a
    destination block names the source block at the same (head, position,
    dimension), in both pools; every other block still names itself; rows
    with an id outside the pool change nothing."""
    nb, H, BS, D = 12, 3, 4, 8
    k0, v0 = _coded_pools(nb, H, BS, D)
    pairs = np.array([[1, 7], [3, 9], [-1, 2], [4, nb], [11, 0]], np.int32)
    k2, v2 = oracle.oracle_copy_blocks(k0, v0, pairs)
    src_of = {7: 1, 9: 3, 0: 11}
    idx = np.indices((H, BS, D))
    for b in range(nb):
        want = src_of.get(b, b)
        code_k = k2[b].astype(np.int64)
        code_v = (-1.0 - v2[b].astype(np.float64)).astype(np.int64)
        for code in (code_k, code_v):
            dd = code % D
            pp = (code // D) % BS
            hh = (code // (D * BS)) % H
            bb = code // (D * BS * H)
            assert (bb == want).all(), b
            assert (hh == idx[0]).all() and (pp == idx[1]).all() and (dd == idx[2]).all()
    assert not np.shares_memory(k2, k0)
    assert (k0 == _coded_pools(nb, H, BS, D)[0]).all()     # inputs untouched


def test_copy_on_write_keeps_the_attention_output():
    """Invariant: pointing a sequence's table at copies of its blocks (the
    copy-on-write step) leaves its attention output bit-identical."""
    rng = np.random.default_rng(57)
    ctx = [37, 64, 5]
    Hq, Hkv, D, BS = 4, 2, 16, 8
    q, seqs = _draw(rng, ctx, Hq, Hkv, D)
    k_pool, v_pool, table, ctx_a = _page(rng, seqs, BS, extra_blocks=20)
    scale = 1.0 / np.sqrt(D)
    base = oracle.oracle_decode(q, k_pool, v_pool, table, ctx_a, scale,
                                Hq // Hkv, BS, "f32")
    used = sorted({int(x) for x in table[table >= 0].ravel()})
    free = [b for b in range(k_pool.shape[0]) if b not in set(used)]
    pairs = np.array(list(zip(used, free[:len(used)])), np.int32)
    k2, v2 = oracle.oracle_copy_blocks(k_pool, v_pool, pairs)
    remap = dict(zip(used, free[:len(used)]))
    table2 = np.vectorize(lambda x: remap.get(int(x), x))(table).astype(np.int32)
    # the originals are overwritten afterwards: only the copies are read
    k2[used] = np.nan
    v2[used] = np.nan
    got = oracle.oracle_decode(q, k2, v2, table2, ctx_a, scale, Hq // Hkv,
                               BS, "f32")
    assert np.array_equal(got, base)


def test_write_then_single_position_decode_round_trip():
    """Round trip: write a token into an empty pool, decode a 1-position
    sequence over it, get the written value back exactly."""
    nb, H, BS, D = 4, 2, 4, 8
    rng = np.random.default_rng(53)
    pk = np.full((nb, H, BS, D), np.nan)
    pv = np.full((nb, H, BS, D), np.nan)
    key = rng.standard_normal((1, H, D))
    val = rng.standard_normal((1, H, D))
    pk, pv = oracle.oracle_cache_write(pk, pv, key, val, np.array([2 * BS]),
                                       BS)
    q = rng.standard_normal((1, 4, D))
    out = oracle.oracle_decode(q, pk, pv, np.array([[2]], dtype=np.int32),
                               np.array([1]), 0.5, 2, BS, "f32")
    for h in range(4):
        assert np.array_equal(out[0, h], val[0, h // 2])


# ---------------------------------------------------------------------------
# storage decoding
# ---------------------------------------------------------------------------

def test_bf16_decoding_matches_torch():
    """Library pin: bf16 bit patterns decode to torch's bfloat16 values."""
    bits = np.arange(0, 2**16, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    ref = ref.to(torch.float64).numpy()
    got = oracle.to_f64(bits, "bf16")
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


# ---------------------------------------------------------------------------
# KV-cache size: values printed on the pages
# ---------------------------------------------------------------------------

def _golden_sizes():
    with open(os.path.join(GOLDEN, "kv_cache_sizes.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_sizes(), ids=lambda c: c["name"])
def test_kv_cache_bytes_printed_values(case):
    n = oracle.kv_cache_bytes(case["n_layers"], case["n_kv_heads"],
                              case["d_head"], case["L"], case["B"],
                              case["n_bytes"])
    if "bytes" in case:
        assert n == case["bytes"]
    if "gib" in case:
        assert n / 2**30 == pytest.approx(case["gib"], abs=0.05)
    if "gb_2dp" in case:
        assert round(n / 1e9, 2) == case["gb_2dp"]
    if "gb_1dp" in case:
        assert round(n / 1e9, 1) == case["gb_1dp"]
    if "kib" in case:
        assert n == case["kib"] * 1024


def test_kv_cache_llama3_half_of_llama2():
    """"Serving", 23.1: LLaMA-3 8B at twice the context needs half the cache
    of LLaMA-2 7B, from having 4 times fewer KV heads."""
    l2 = oracle.kv_cache_bytes(32, 32, 128, 4096, 1, 2)
    l3 = oracle.kv_cache_bytes(32, 8, 128, 8192, 1, 2)
    assert 2 * l3 == l2


def test_llama2_pool_is_two_gib_per_layer_of_32_sequences():
    """The MHA decode batch (32 sequences x 4096 positions, one layer, fp16)
    holds exactly 2^31 bytes of K+V: the closed form at n_layers=1, B=32."""
    assert oracle.kv_cache_bytes(1, 32, 128, 4096, 32, 2) == 2**31


# ---------------------------------------------------------------------------
# Mutation tests: a planted mistake in the oracle must trip a pin
# ---------------------------------------------------------------------------

def _run_pins():
    """Run the decode pins; return True when all pass."""
    try:
        for args in CASES:
            test_paged_equals_contiguous_sdpa(*args)
        test_stress_large_logits_equal_sdpa()
        for P in (4, 12):
            test_partition_merge_equals_unsplit(P)
    except AssertionError:
        return False
    except (FloatingPointError, ValueError, IndexError):
        return False
    return True


def test_pins_pass_unmutated():
    assert _run_pins()


MUTANTS = {
    "gqa_mapping_modulo": ("_kv_head", lambda h, G: h % G),
    "block_offset_off_by_one": (
        "_token_location",
        lambda row, t, bs: (row[t // bs].astype(np.int64), (t + 1) % bs)),
    "table_index_uses_offset": (
        "_token_location",
        lambda row, t, bs: (row[t % len(row)].astype(np.int64), t % bs)),
    "scale_dropped": ("_logits", lambda q, k, s: k @ q),
    "sign_flipped": ("_logits", lambda q, k, s: -s * (k @ q)),
    "softmax_without_max": ("_softmax",
                            lambda s: np.exp(s) / np.exp(s).sum()),
    "softmax_unnormalised": ("_softmax", lambda s: np.exp(s - s.max())),
    "values_reversed": ("_weighted_sum", lambda p, v: p @ v[::-1]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(pa_oracle, attr, fn)
    with np.errstate(all="ignore"):
        assert not _run_pins(), f"mutant {name} survived every pin"


def test_planted_merge_mistake_is_caught(monkeypatch):
    """Dropping the l_p weight from the merge must fail the merge pin."""
    def bad_merge(m, l, o, cl, P):
        B, Hq, PM, D = o.shape
        out = np.zeros((B, Hq, D))
        for b in range(B):
            n_p = -(-int(cl[b]) // P)
            for h in range(Hq):
                if n_p:
                    w = np.exp(m[b, h, :n_p] - m[b, h, :n_p].max())
                    out[b, h] = (w[:, None] * o[b, h, :n_p]).sum(0) / w.sum()
        return out
    monkeypatch.setattr(oracle, "oracle_merge", bad_merge)
    with pytest.raises(AssertionError):
        test_partition_merge_equals_unsplit(4)


def test_planted_cache_write_mistake_is_caught(monkeypatch):
    """Swapping block and offset in the write must fail the slot-view pin."""
    def bad_write(k_pool, v_pool, key, value, slots, bs):
        k_out, v_out = k_pool.copy(), v_pool.copy()
        for i, s in enumerate(slots.tolist()):
            if s >= 0:
                k_out[s % k_pool.shape[0], :, (s // k_pool.shape[0]) % bs] = key[i]
                v_out[s % k_pool.shape[0], :, (s // k_pool.shape[0]) % bs] = value[i]
        return k_out, v_out
    monkeypatch.setattr(oracle, "oracle_cache_write", bad_write)
    with pytest.raises(AssertionError):
        test_cache_write_matches_flat_slot_view("f32")


def test_planted_copy_blocks_mistake_is_caught(monkeypatch):
    """Copying the destination onto the source, or only the K pool, must
    fail the code pin."""
    real = oracle.oracle_copy_blocks

    def reversed_copy(k_pool, v_pool, pairs):
        return real(k_pool, v_pool, np.asarray(pairs)[:, ::-1].copy())

    def k_only(k_pool, v_pool, pairs):
        k2, _ = real(k_pool, v_pool, pairs)
        return k2, v_pool.copy()

    for bad in (reversed_copy, k_only):
        monkeypatch.setattr(oracle, "oracle_copy_blocks", bad)
        with pytest.raises(AssertionError):
            test_copy_blocks_moves_whole_blocks()


def test_planted_multi_query_mistake_is_caught(monkeypatch):
    """A mask that lets every token see all positions, one that hides the
    token's own position, or the tokens taken in reverse order must fail the
    SDPA pin."""
    real_row = pa_oracle.oracle_decode_row

    def make(shift):
        def bad(q, k_pool, v_pool, block_table, context_lens, scale, G, BS,
                dtype, rows=None):
            B, k, Hq, D = q.shape
            out = np.zeros((B, k, Hq, D))
            for b in range(B):
                for j in range(k):
                    for h in range(Hq):
                        n = int(context_lens[b])
                        stop = {"all": n, "own": n - k + j,
                                "rev": n - j}[shift]
                        if stop <= 0:
                            continue
                        out[b, j, h], _ = real_row(
                            q[:, j], k_pool, v_pool, block_table,
                            context_lens, scale, G, BS, dtype, b, h,
                            stop=stop)
            return out
        return bad

    for shift in ("all", "own", "rev"):
        monkeypatch.setattr(oracle, "oracle_decode_multi", make(shift))
        with pytest.raises(AssertionError):
            test_multi_query_equals_masked_sdpa([33, 64, 4], 8, 2, 16, 16, 4)
