"""pa_decode_shared_prefix through the C ABI (needs an MI355X): the shared
partitions of a common prefix computed for several sequences per work item,
then pa_reduce.  The output must be within the stated tolerance of the fp64
oracle, the folded cache write bit-exact, the workspace of the shared
partitions consistent with the oracle's per-partition statistics, and the
result run-to-run deterministic.  Covers both element types, both head
widths, block sizes 8-64, group sizes that put 16, 4, 2 and 1 sequences in a
work item (and a group split over two column chunks), a prefix that is not
a whole number of partitions, a batch that is not a whole number of groups,
sequences that end inside the prefix, invalid lengths, seeded random shapes,
and the full shared-prefix batch at both block sizes and both
partition sizes, every row."""

import numpy as np
import pytest
import torch

import oracle
from helpers import (TOL, DeviceBatch, as_f64, from_dev, note, oracle_out,
                     full_batch, oracle_pools_after_write, out_bound)
from paged_kv_cache_222_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_222_amd as pa
    pa.load()
    return pa


def _run(pa, d, P, prefix_len, *, write, name):
    B, Hq, D = d.q.shape
    pm = max(1, -(-int(d.context_lens.max().item()) // P))
    ws = pa.partition_workspace(B, Hq, D, pm)
    for t in ws:
        t.fill_(float("nan"))
    note(f"pa_decode_shared_prefix {name} P={P} prefix={prefix_len} "
         f"write={write}")
    kw = dict(key_new=d.key_new, value_new=d.value_new) if write else {}
    pa.pa_decode_shared_prefix(*ws, d.q, d.k_pool, d.v_pool, d.block_table,
                               d.context_lens, partition_size=P,
                               prefix_len=prefix_len, scale=d.scale, **kw)
    out = d.empty_out()
    pa.pa_reduce(out, *ws, d.context_lens, partition_size=P)
    torch.cuda.synchronize()
    return out, ws


CASES = [  # dtype, D, BS, Hkv, G, P, prefix, batch
    ("bf16", 128, 16, 2, 4, 64, 192, 13),    # 4 sequences per item, 1 left over
    ("f16", 64, 8, 1, 6, 64, 100, 7),        # 2 per item; prefix not whole partitions
    ("bf16", 128, 32, 2, 1, 128, 256, 21),   # MHA: 16 per item
    ("f16", 128, 64, 1, 8, 256, 384, 5),     # 2 per item; 1.5 partitions of prefix
    ("bf16", 64, 16, 3, 16, 16, 48, 6),      # 1 per item
    ("f16", 64, 16, 1, 20, 32, 64, 4),       # the group spans two column chunks
]


@pytest.mark.parametrize("dtype,D,BS,Hkv,G,P,prefix,B", CASES)
def test_shared_prefix_matches_oracle(pa, dtype, D, BS, Hkv, G, P, prefix, B):
    rng = np.random.default_rng(D + G + P + B)
    # suffixes from one position (only the new token) to several partitions
    suffix = rng.integers(1, 4 * P, size=B)
    suffix[0] = 1
    plen = prefix - prefix % BS     # the shared blocks: whole blocks only
    ctx = [plen + int(s) for s in suffix]
    w = wl.make_custom(ctx, n_q_heads=Hkv * G, n_kv_heads=Hkv, d_head=D,
                       block_size=BS, dtype=dtype, seed=int(B + P),
                       prefix_len=plen)
    d = DeviceBatch(w)
    name = f"{dtype} D{D} BS{BS} G{G}"
    out, ws = _run(pa, d, P, plen, write=True, name=name)
    k_ref, v_ref = oracle_pools_after_write(w)
    assert from_dev(d.k_pool).tobytes() == k_ref.tobytes()
    assert from_dev(d.v_pool).tobytes() == v_ref.tobytes()
    ref = oracle_out(w, k_ref, v_ref)
    err = np.abs(as_f64(out) - ref)
    assert (err <= out_bound(ref, dtype)).all(), err.max()
    # every partition of every row was written (the workspace was NaN)
    gm, gl, go = (from_dev(t).astype(np.float64) for t in ws)
    for b in range(B):
        n_p = -(-ctx[b] // P)
        assert np.isfinite(gm[b, :, :n_p]).all()
        assert np.isfinite(go[b, :, :n_p]).all()
    # the shared partitions against the oracle's statistics
    c = w.cfg
    rows = [(b, h) for b in range(B) for h in range(c.n_q_heads)]
    m, l, o = oracle.oracle_partitions(
        w.q, k_ref, v_ref, w.block_table, w.context_lens, w.scale,
        c.gqa_group, c.block_size, c.dtype, P, max_partitions=gm.shape[2],
        rows=rows)
    lse_tol = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}[dtype]
    for b, h in rows:
        n_p = -(-ctx[b] // P)
        lse_ref = m[b, h, :n_p] + np.log(l[b, h, :n_p])
        lse_gpu = gm[b, h, :n_p] + np.log(gl[b, h, :n_p])
        assert np.max(np.abs(lse_gpu - lse_ref)) < lse_tol
        assert (gm[b, h, :n_p] <= m[b, h, :n_p] + 1e-5).all()
        assert (gm[b, h, :n_p] >= m[b, h, :n_p] - 8 * np.log(2) - 1e-5).all()
        assert np.max(np.abs(go[b, h, :n_p] - o[b, h, :n_p])) <= TOL[dtype]


def test_write_is_the_one_of_decode_step(pa):
    """With the new rows, the pools equal those of pa_decode_step bit for
    bit, and the output agrees with it within the tolerance."""
    ctx = [256 + s for s in (1, 5, 70, 129, 300, 2, 64, 17, 33)]
    w = wl.make_custom(ctx, n_q_heads=8, n_kv_heads=2, d_head=128,
                       block_size=16, dtype="bf16", seed=5, prefix_len=256)
    d1, d2 = DeviceBatch(w), DeviceBatch(w)
    out1, _ = _run(pa, d1, 64, 256, write=True, name="prefix")
    B, Hq, D = d2.q.shape
    ws = pa.partition_workspace(B, Hq, D, -(-max(ctx) // 64))
    note("pa_decode_step reference P=64")
    pa.pa_decode_step(*ws, d2.key_new, d2.value_new, d2.q, d2.k_pool,
                      d2.v_pool, d2.block_table, d2.context_lens,
                      partition_size=64, scale=d2.scale)
    out2 = d2.empty_out()
    pa.pa_reduce(out2, *ws, d2.context_lens, partition_size=64)
    torch.cuda.synchronize()
    assert from_dev(d1.k_pool).tobytes() == from_dev(d2.k_pool).tobytes()
    assert from_dev(d1.v_pool).tobytes() == from_dev(d2.v_pool).tobytes()
    assert np.max(np.abs(as_f64(out1) - as_f64(out2))) <= TOL["bf16"]


def test_sequences_ending_inside_the_prefix(pa):
    """A sequence shorter than the shared prefix (its table still names the
    shared blocks) limits the shared partitions to those before its end;
    attention only, since its new token would land in a shared block."""
    ctx = [600, 700, 650, 900, 610, 820]
    w = wl.make_custom(ctx, n_q_heads=8, n_kv_heads=2, d_head=128,
                       block_size=16, dtype="bf16", seed=7, prefix_len=512)
    d = DeviceBatch(w)
    k_ref, v_ref = oracle_pools_after_write(w)
    note("write the new rows with pa_cache_write")
    pa.pa_cache_write(d.key_new, d.value_new, d.k_pool, d.v_pool,
                      d.slot_mapping)
    short = np.array(ctx)
    short[2] = 200          # ends inside partition 3 of 64 (prefix: 8)
    short[4] = 64           # ends exactly at the first partition's end
    d.context_lens.copy_(torch.from_numpy(short.astype(np.int32)))
    w.context_lens = short.astype(np.int32)
    out, _ = _run(pa, d, 64, 512, write=False, name="short rows")
    ref = oracle_out(w, k_ref, v_ref)
    err = np.abs(as_f64(out) - ref)
    assert (err <= out_bound(ref, "bf16")).all(), err.max()


def test_invalid_lengths_give_nan_rows_only_there(pa):
    ctx = [300, 400, 350, 500, 320, 330, 341, 290]
    w = wl.make_custom(ctx, n_q_heads=8, n_kv_heads=2, d_head=64,
                       block_size=16, dtype="f16", seed=8, prefix_len=256)
    d = DeviceBatch(w)
    note("pa_cache_write before the invalid-length case")
    pa.pa_cache_write(d.key_new, d.value_new, d.k_pool, d.v_pool,
                      d.slot_mapping)
    good, _ = _run(pa, d, 64, 256, write=False, name="valid")
    good = as_f64(good)
    bad = np.array(ctx, dtype=np.int32)
    bad[1] = -3
    bad[6] = w.max_blocks * 16 + 1
    d.context_lens.copy_(torch.from_numpy(bad))
    out, _ = _run(pa, d, 64, 256, write=False, name="invalid lengths")
    out = as_f64(out)
    assert np.isnan(out[1]).all() and np.isnan(out[6]).all()
    for b in (0, 2, 3, 4, 5, 7):
        assert np.isfinite(out[b]).all()
        assert np.max(np.abs(out[b] - good[b])) <= TOL["f16"]


def test_run_to_run_determinism(pa):
    ctx = [1024 + s for s in range(1, 200, 7)]
    w = wl.make_custom(ctx, n_q_heads=32, n_kv_heads=8, d_head=128,
                       block_size=16, dtype="bf16", seed=9, prefix_len=1024)
    outs = []
    for _ in range(2):
        d = DeviceBatch(w)
        out, ws = _run(pa, d, 256, 1024, write=True, name="determinism")
        outs.append((from_dev(out), [from_dev(t) for t in ws]))
    assert outs[0][0].tobytes() == outs[1][0].tobytes()
    for a, b in zip(outs[0][1], outs[1][1]):
        assert np.array_equal(np.nan_to_num(a, nan=7.0),
                              np.nan_to_num(b, nan=7.0))


@pytest.mark.parametrize("P", [512, 2048])
@pytest.mark.parametrize("bs", [16, 32])
def test_full_shared_prefix_batch(pa, bs, P):
    """The full shared-prefix batch (B 256, 1.3 M positions) at the
    batch's own 512-token partitions and at 2048, both block sizes: the
    pools bit for bit after the folded write, and every output element of
    every (sequence, head) within the stated bf16 tolerance."""
    w, k_ref, v_ref, ref = full_batch("shared-prefix", bs)
    d = DeviceBatch(w)
    out, ws = _run(pa, d, P, w.cfg.prefix_len, write=True,
                   name=f"shared-prefix bs{bs}")
    assert from_dev(d.k_pool).tobytes() == k_ref.tobytes()
    assert from_dev(d.v_pool).tobytes() == v_ref.tobytes()
    got = as_f64(out)
    err = float(np.max(np.abs(got - ref)))
    print(f"shared-prefix bs{bs} P{P}: max err {err:.3g} over all rows")
    assert err <= TOL["bf16"]
    del d, out, ws
    torch.cuda.empty_cache()


def _step_reference(pa, w, P):
    """pa_decode_step + pa_reduce on a fresh upload of w."""
    d = DeviceBatch(w)
    B, Hq, D = d.q.shape
    ws = pa.partition_workspace(B, Hq, D, -(-int(w.context_lens.max()) // P))
    note(f"pa_decode_step reference P={P}")
    pa.pa_decode_step(*ws, d.key_new, d.value_new, d.q, d.k_pool, d.v_pool,
                      d.block_table, d.context_lens, partition_size=P,
                      scale=d.scale)
    out = d.empty_out()
    pa.pa_reduce(out, *ws, d.context_lens, partition_size=P)
    torch.cuda.synchronize()
    return d, out


def test_zero_prefix_is_decode_step_bit_for_bit(pa):
    ctx = [300 + 37 * i for i in range(11)]
    w = wl.make_custom(ctx, n_q_heads=32, n_kv_heads=8, d_head=128,
                       block_size=16, dtype="bf16", seed=21, prefix_len=256)
    d1 = DeviceBatch(w)
    out1, _ = _run(pa, d1, 128, 0, write=True, name="prefix_len 0")
    d2, out2 = _step_reference(pa, w, 128)
    assert from_dev(out1).tobytes() == from_dev(out2).tobytes()
    assert from_dev(d1.k_pool).tobytes() == from_dev(d2.k_pool).tobytes()


@pytest.mark.parametrize("case", ["f32", "batch over 1024"])
def test_paths_without_shared_items(pa, case):
    """fp32 (vector-ALU kernel) and batches beyond the in-kernel plan run
    every row through its own table: the result of pa_decode_step, bit for
    bit, and within the tolerance of the oracle."""
    if case == "f32":
        ctx = [70, 90, 65, 130, 81]
        w = wl.make_custom(ctx, n_q_heads=4, n_kv_heads=2, d_head=64,
                           block_size=16, dtype="f32", seed=22, prefix_len=64)
        P = 32
    else:
        rng = np.random.default_rng(23)
        ctx = [64 + int(s) for s in rng.integers(1, 40, size=1030)]
        w = wl.make_custom(ctx, n_q_heads=4, n_kv_heads=1, d_head=64,
                           block_size=16, dtype="f16", seed=23, prefix_len=64)
        P = 32
    d1 = DeviceBatch(w)
    out1, _ = _run(pa, d1, P, 64, write=True, name=case)
    _, out2 = _step_reference(pa, w, P)
    assert from_dev(out1).tobytes() == from_dev(out2).tobytes()
    k_ref, v_ref = oracle_pools_after_write(w)
    assert from_dev(d1.k_pool).tobytes() == k_ref.tobytes()
    ref = oracle_out(w, k_ref, v_ref)
    err = np.abs(as_f64(out1) - ref)
    assert (err <= out_bound(ref, w.cfg.dtype)).all()


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes_against_oracle(pa, seed):
    """Seeded random batches: batch size, group size, head width, block
    size, partition size and prefix length all drawn, so the plan sees
    shared items fewer than, equal to and more than the full partitions,
    groups that do not divide the batch, and prefixes of zero to several
    partitions."""
    rng = np.random.default_rng(1000 + seed)
    dtype = ["bf16", "f16"][seed % 2]
    D = [64, 128][int(rng.integers(0, 2))]
    BS = [8, 16, 32][int(rng.integers(0, 3))]
    Hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    P = BS * int(rng.integers(1, 9))
    B = int(rng.integers(1, 60))
    plen = BS * int(rng.integers(0, 30))
    ctx = [plen + int(s) for s in rng.integers(1, 5 * P, size=B)]
    w = wl.make_custom(ctx, n_q_heads=Hkv * G, n_kv_heads=Hkv, d_head=D,
                       block_size=BS, dtype=dtype, seed=2000 + seed,
                       prefix_len=plen)
    d = DeviceBatch(w)
    name = f"random seed {seed}: {dtype} D{D} BS{BS} Hkv{Hkv} G{G} B{B}"
    out, _ = _run(pa, d, P, plen, write=True, name=name)
    k_ref, v_ref = oracle_pools_after_write(w)
    assert from_dev(d.k_pool).tobytes() == k_ref.tobytes()
    ref = oracle_out(w, k_ref, v_ref)
    err = np.abs(as_f64(out) - ref)
    assert (err <= out_bound(ref, dtype)).all(), \
        (name, float(err.max()))


def _prefix_batch(dtype="bf16", D=128, BS=16, spare=64, seed=51):
    ctx = [512 + s for s in (40, 300, 7, 129, 260, 64, 1, 90, 200, 33, 17,
                             150)]
    return wl.make_custom(ctx, n_q_heads=8, n_kv_heads=2, d_head=D,
                          block_size=BS, dtype=dtype, seed=seed,
                          prefix_len=512,
                          pool_blocks=sum(-(-c // BS) for c in ctx) - 32 * 11
                          + spare)


def test_rows_not_sharing_the_prefix_get_nan(pa):
    """G = 4 puts 4 sequences in a shared item (P 128: prefix partitions
    0-3).  Sequence 5 (second of group 1) and sequence 8 (first of group 2)
    point one block of shared partition 2 at a private copy of it.  The item
    reads its first sequence's table and checks the others against it:
    sequence 5 is NaN; in group 2 the others (9, 10, 11) differ from
    sequence 8 and are NaN, sequence 8 is correct; every other row matches
    the oracle, since a copy of a block holds the same values."""
    w = _prefix_batch()
    bs, P = 16, 128
    free = sorted(set(range(w.n_blocks)) - set(w.block_table[w.block_table >= 0].tolist()))
    j_shared = 2 * P // bs + 3          # a block of partition 2
    for s, fb in ((5, free[0]), (8, free[1])):
        src = int(w.block_table[s, j_shared])
        w.k_pool[fb] = w.k_pool[src]
        w.v_pool[fb] = w.v_pool[src]
        w.block_table[s, j_shared] = fb
    d = DeviceBatch(w)
    out, _ = _run(pa, d, P, 512, write=True, name="mismatched tables")
    k_ref, v_ref = oracle_pools_after_write(w)
    assert from_dev(d.k_pool).tobytes() == k_ref.tobytes()
    ref = oracle_out(w, k_ref, v_ref)
    got = as_f64(out)
    nan_rows = {5, 9, 10, 11}
    for b in range(len(w.context_lens)):
        if b in nan_rows:
            assert np.isnan(got[b]).all(), b
        else:
            assert (np.abs(got[b] - ref[b]) <= out_bound(ref[b], "bf16")).all(), b


def test_mismatch_past_the_first_512_pairs_is_found(pa):
    """G = 1 puts 16 sequences in a shared item; with blocks of 8 and 1024-
    position partitions an item has 15 x 128 = 1920 (sequence, block) pairs
    to check, past the two per thread the item keeps in registers.
    Sequence 2 differs at block 10 of partition 0 (pair 138) and sequence 15
    at its last block (pair 1919): both NaN, every other row the oracle's."""
    bs, P, plen = 8, 1024, 2048
    ctx = [plen + 1 + 8 * (i % 5) + i for i in range(18)]
    w = wl.make_custom(ctx, n_q_heads=2, n_kv_heads=2, d_head=128,
                       block_size=bs, dtype="bf16", seed=61,
                       prefix_len=plen,
                       pool_blocks=sum(-(-c // bs) for c in ctx)
                       - (plen // bs) * (len(ctx) - 1) + 16)
    free = sorted(set(range(w.n_blocks)) -
                  set(w.block_table[w.block_table >= 0].tolist()))
    for s, j, fb in ((2, 10, free[0]), (15, P // bs - 1, free[1])):
        src = int(w.block_table[s, j])
        w.k_pool[fb] = w.k_pool[src]
        w.v_pool[fb] = w.v_pool[src]
        w.block_table[s, j] = fb
    d = DeviceBatch(w)
    out, _ = _run(pa, d, P, plen, write=True, name="mismatch past 512 pairs")
    k_ref, v_ref = oracle_pools_after_write(w)
    ref = oracle_out(w, k_ref, v_ref)
    got = as_f64(out)
    for b in range(len(ctx)):
        if b in (2, 15):
            assert np.isnan(got[b]).all(), b
        else:
            assert (np.abs(got[b] - ref[b]) <= out_bound(ref[b], "bf16")).all(), b


def test_private_copy_outside_shared_items_is_correct(pa):
    """A row that points a prefix block at a copy outside every shared
    partition reads it through its own table: the oracle's result."""
    w = _prefix_batch(seed=52)
    bs, P = 16, 384      # one shared partition (0-383); 384-511 are private
    free = sorted(set(range(w.n_blocks)) - set(w.block_table[w.block_table >= 0].tolist()))
    j = 400 // bs
    src = int(w.block_table[6, j])
    w.k_pool[free[0]] = w.k_pool[src]
    w.v_pool[free[0]] = w.v_pool[src]
    w.block_table[6, j] = free[0]
    d = DeviceBatch(w)
    out, _ = _run(pa, d, P, 512, write=True, name="private copy")
    k_ref, v_ref = oracle_pools_after_write(w)
    ref = oracle_out(w, k_ref, v_ref)
    err = np.abs(as_f64(out) - ref)
    assert (err <= out_bound(ref, "bf16")).all(), float(np.nanmax(err))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_new_token_inside_the_prefix(pa, dtype):
    """With a folded write, a sequence whose new token would land in the
    shared positions (n - 1 < prefix_len) is not written and its row is
    NaN; every other sequence is written and matches the oracle.  bf16 runs
    the shared items, fp32 the fallback with its own write kernel."""
    D = 64 if dtype == "f32" else 128
    w = _prefix_batch(dtype=dtype, D=D, seed=53)
    short = w.context_lens.copy()
    short[3] = 300          # its slot would be position 299, a shared block
    short[7] = 512          # position 511: the last shared position
    w.context_lens = short
    d = DeviceBatch(w)
    P = 128
    out, _ = _run(pa, d, P, 512, write=True, name=f"in-prefix write {dtype}")
    slots = w.slot_mapping.copy()
    slots[3] = slots[7] = -1                   # not written
    k_ref, v_ref = oracle.oracle_cache_write(w.k_pool, w.v_pool, w.key_new,
                                             w.value_new, slots,
                                             w.cfg.block_size)
    assert from_dev(d.k_pool).tobytes() == k_ref.tobytes()
    assert from_dev(d.v_pool).tobytes() == v_ref.tobytes()
    got = as_f64(out)
    assert np.isnan(got[3]).all() and np.isnan(got[7]).all()
    keep = [b for b in range(len(short)) if b not in (3, 7)]
    ref = oracle_out(w, k_ref, v_ref, [(b, h) for b in keep
                                       for h in range(w.q.shape[1])])
    err = np.abs(got[keep] - ref[keep])
    assert (err <= out_bound(ref[keep], dtype)).all()
