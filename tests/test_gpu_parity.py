"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X).

Every output element is compared with the oracle on the same seeded inputs:
bit for bit for the cache write, within the stated max-abs-error for
attention.  The five decode batches run at full size, every row; a matrix of small batches covers every element type, head
width, block size and group size with ragged lengths; the invariants and edge
cases of the method close the file.
"""

import numpy as np
import pytest
import torch

import oracle
from helpers import (TOL, DeviceBatch, as_f64, from_dev, note, oracle_out,
                     full_batch, oracle_pools_after_write, out_bound, to_dev)
from paged_kv_cache_222_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_222_amd as pa
    pa.load()
    return pa


def sync():
    torch.cuda.synchronize()


def run_write(pa, d, name=""):
    note(f"pa_cache_write {name}")
    pa.pa_cache_write(d.key_new, d.value_new, d.k_pool, d.v_pool,
                      d.slot_mapping)
    sync()


def run_decode(pa, d, name=""):
    note(f"pa_decode {name}")
    out = d.empty_out()
    pa.pa_decode(out, d.q, d.k_pool, d.v_pool, d.block_table, d.context_lens,
                 scale=d.scale)
    sync()
    return out


def run_partitioned(pa, d, partition_size=None, max_partitions=None, name=""):
    """pa_decode_partitioned + pa_reduce."""
    P = partition_size or d.partition_size
    pm = max_partitions or max(1, -(-int(d.w.context_lens.max()) // P))
    B, Hq, D = d.q.shape
    ws = pa.partition_workspace(B, Hq, D, pm)
    for t in ws:
        t.fill_(float("nan"))
    note(f"pa_decode_partitioned+pa_reduce {name} P={P} PMAX={pm}")
    pa.pa_decode_partitioned(*ws, d.q, d.k_pool, d.v_pool, d.block_table,
                             d.context_lens, partition_size=P, scale=d.scale)
    out = d.empty_out()
    pa.pa_reduce(out, *ws, d.context_lens, partition_size=P)
    sync()
    return out, ws


def max_err(got, ref, rows=None):
    if rows is not None:
        idx = tuple(np.array(rows).T)
        got, ref = got[idx], ref[idx]
    return float(np.max(np.abs(got - ref)))


# ---------------------------------------------------------------------------
# the five decode batches at full size
# ---------------------------------------------------------------------------

FULL = [("tiny", {}), ("qwen2.5-1.5b", {}), ("llama2-7b", {}),
        ("llama3-8b", {}), ("shared-prefix", {}),
        ("shared-prefix", {"block_size": 32})]


@pytest.mark.parametrize("name,kw", FULL,
                         ids=[n + ("-bs32" if k else "") for n, k in FULL])
def test_full_batch_step(pa, name, kw):
    w, k_ref, v_ref, ref = full_batch(name, kw.get("block_size"))
    d = DeviceBatch(w)
    # 1. cache write: the whole pool, bit for bit
    run_write(pa, d, name)
    assert from_dev(d.k_pool).tobytes() == k_ref.tobytes()
    assert from_dev(d.v_pool).tobytes() == v_ref.tobytes()
    # 2. decode over the written pool: every (sequence, head)
    rows = None
    tol = TOL[w.cfg.dtype]
    e1 = max_err(as_f64(run_decode(pa, d, name)), ref, rows)
    out2, ws = run_partitioned(pa, d, name=name)
    e2 = max_err(as_f64(out2), ref, rows)
    print(f"{name} {kw}: single-pass err {e1:.3g}, partitioned err {e2:.3g}")
    assert e1 <= tol and e2 <= tol
    # 3. the partition workspace on a few rows
    c = w.cfg
    rng = np.random.default_rng(2)
    B, Hq = w.q.shape[:2]
    sample = [(int(b), int(h)) for b, h in
              zip(rng.integers(0, B, 6), rng.integers(0, Hq, 6))]
    m, l, o = oracle.oracle_partitions(
        w.q, k_ref, v_ref, w.block_table, w.context_lens, w.scale,
        c.gqa_group, c.block_size, c.dtype, c.partition_size,
        max_partitions=ws[0].shape[2], rows=sample)
    gm, gl, go = (from_dev(t).astype(np.float64) for t in ws)
    # The softmax weights are rounded to the storage type before they
    # multiply V (fp32 kept for fp32 data), and l sums the rounded weights:
    # each weight is off by at most half an ulp (2^-9 bf16, 2^-12 fp16), so
    # ln(l) moves by at most that much; the normalised partial output is a
    # convex combination like the final one and gets the final tolerance.
    lse_tol = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 1e-5}[c.dtype]
    for b, h in sample:
        n_p = -(-int(w.context_lens[b]) // c.partition_size)
        lse_ref = m[b, h, :n_p] + np.log(l[b, h, :n_p])
        lse_gpu = gm[b, h, :n_p] + np.log(gl[b, h, :n_p])
        assert np.max(np.abs(lse_gpu - lse_ref)) < lse_tol
        assert (gm[b, h, :n_p] <= m[b, h, :n_p] + 1e-5).all()
        assert (gm[b, h, :n_p] >= m[b, h, :n_p] - 8 * np.log(2) - 1e-5).all()
        assert np.max(np.abs(go[b, h, :n_p] - o[b, h, :n_p])) <= tol


# ---------------------------------------------------------------------------
# small batches: every element type, head width, block size and group size
# ---------------------------------------------------------------------------

RAGGED = [1, 2, 7, 8, 9, 15, 16, 17, 33, 64, 100, 129, 257, 513, 1000]
GROUPS = [1, 2, 3, 4, 5, 6, 7, 8, 12, 16]
MATRIX = [(dt, D, BS, GROUPS[i % len(GROUPS)])
          for i, (dt, D, BS) in enumerate(
              (dt, D, BS) for dt in ("f32", "f16", "bf16") for D in (64, 128)
              for BS in (8, 16, 32, 64))]
MATRIX += [("bf16", 128, 16, G) for G in (1, 2, 3, 5, 6, 7, 8, 16, 32)]


def _check_small(pa, w, partition_sizes):
    d = DeviceBatch(w)
    run_write(pa, d, "small")
    k_ref, v_ref = oracle_pools_after_write(w)
    assert from_dev(d.k_pool).tobytes() == k_ref.tobytes()
    ref = oracle_out(w, k_ref, v_ref)
    bound = out_bound(ref, w.cfg.dtype)
    got = as_f64(run_decode(pa, d, "small"))
    assert (np.abs(got - ref) <= bound).all(), np.max(np.abs(got - ref))
    for P in partition_sizes:
        got, _ = run_partitioned(pa, d, partition_size=P)
        assert (np.abs(as_f64(got) - ref) <= bound).all(), P


@pytest.mark.parametrize("dt,D,BS,G", MATRIX,
                         ids=[f"{a}-d{b}-bs{c}-g{g}" for a, b, c, g in MATRIX])
def test_small_batch_matrix(pa, dt, D, BS, G):
    n_kv = 2 if G <= 8 else 1
    w = wl.make_custom(RAGGED, n_q_heads=n_kv * G, n_kv_heads=n_kv, d_head=D,
                       block_size=BS, dtype=dt, seed=G + D + BS,
                       pool_blocks=None)
    _check_small(pa, w, sorted({BS, 64 if 64 % BS == 0 else BS, 512}))


def test_many_kv_heads_long_context(pa):
    """32 KV heads, fp16, 3000-position contexts: many windows of the
    block table in single-pass mode."""
    w = wl.make_custom([3000, 2049, 5], n_q_heads=32, n_kv_heads=32,
                       d_head=128, block_size=16, dtype="f16", seed=9,
                       std=0.5)
    _check_small(pa, w, [256, 4096])


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_single_position_is_exact(pa, dt):
    """ctx = 1: the softmax weight is exactly 1, so out = v_0 bit for bit."""
    w = wl.make_custom([1, 1, 1], n_q_heads=8, n_kv_heads=2, d_head=128,
                       block_size=16, dtype=dt, seed=3)
    d = DeviceBatch(w)
    run_write(pa, d)
    expect = np.repeat(from_dev(d.value_new), 4, axis=1)   # [B, Hq, D]
    assert from_dev(run_decode(pa, d)).tobytes() == expect.tobytes()
    out, _ = run_partitioned(pa, d, partition_size=16)
    assert from_dev(out).tobytes() == expect.tobytes()


def test_uniform_values_give_ones(pa):
    w = wl.make_custom([5, 300, 1000], n_q_heads=8, n_kv_heads=2, d_head=128,
                       block_size=16, dtype="bf16", seed=4)
    d = DeviceBatch(w)
    one = torch.ones((), dtype=torch.bfloat16, device="cuda")
    d.v_pool.copy_(one.expand_as(d.v_pool))
    d.value_new.copy_(one.expand_as(d.value_new))
    run_write(pa, d)
    assert np.max(np.abs(as_f64(run_decode(pa, d)) - 1.0)) <= TOL["bf16"]
    out, _ = run_partitioned(pa, d, partition_size=64)
    assert np.max(np.abs(as_f64(out) - 1.0)) <= TOL["bf16"]


def test_block_relabelling_is_bit_identical(pa):
    """Permuting physical block ids (pool rows and table entries together)
    leaves both paths' outputs unchanged bit for bit."""
    w = wl.make_workload("llama3-8b", seed=5, batch=16)
    d = DeviceBatch(w)
    run_write(pa, d)
    a1 = from_dev(run_decode(pa, d))
    a2 = from_dev(run_partitioned(pa, d)[0])
    rng = np.random.default_rng(8)
    pi = rng.permutation(w.n_blocks)
    pit = torch.from_numpy(pi).to("cuda")
    k2 = torch.empty_like(d.k_pool)
    v2 = torch.empty_like(d.v_pool)
    k2[pit] = d.k_pool
    v2[pit] = d.v_pool
    d.k_pool, d.v_pool = k2, v2
    tbl = w.block_table
    d.block_table = to_dev(np.where(tbl >= 0, pi[np.maximum(tbl, 0)], -1)
                           .astype(np.int32))
    assert from_dev(run_decode(pa, d)).tobytes() == a1.tobytes()
    assert from_dev(run_partitioned(pa, d)[0]).tobytes() == a2.tobytes()


def test_run_to_run_determinism(pa):
    w = wl.make_workload("qwen2.5-1.5b", seed=6, batch=16)
    d = DeviceBatch(w)
    run_write(pa, d)
    outs = [from_dev(run_decode(pa, d)).tobytes() for _ in range(3)]
    parts = [from_dev(run_partitioned(pa, d)[0]).tobytes() for _ in range(3)]
    assert len(set(outs)) == 1 and len(set(parts)) == 1


def test_shared_prefix_rows_are_identical(pa):
    """Sequences with the same table prefix, equal suffix contents and equal
    queries decode to identical outputs."""
    w = wl.make_custom([2048 + 300, 2048 + 300, 2048 + 77], n_q_heads=32,
                       n_kv_heads=8, d_head=128, block_size=16, dtype="bf16",
                       seed=7, prefix_len=2048)
    k, v, tbl = w.k_pool.copy(), w.v_pool.copy(), w.block_table
    for j in range(128, 128 + -(-300 // 16)):          # copy row 0's suffix
        k[tbl[1, j]] = k[tbl[0, j]]
        v[tbl[1, j]] = v[tbl[0, j]]
    w.k_pool, w.v_pool = k, v
    w.q[1] = w.q[0]
    w.key_new[1], w.value_new[1] = w.key_new[0], w.value_new[0]
    d = DeviceBatch(w)
    run_write(pa, d)
    out = from_dev(run_decode(pa, d))
    assert out[0].tobytes() == out[1].tobytes()
    part = from_dev(run_partitioned(pa, d)[0])
    assert part[0].tobytes() == part[1].tobytes()


def test_sharp_logits(pa):
    """Queries scaled by 8 (exactly, a power of two) make the softmax sharp;
    the running-max rescaling keeps the result within tolerance."""
    w = wl.make_custom([40, 700, 2500], n_q_heads=8, n_kv_heads=2, d_head=128,
                       block_size=16, dtype="f16", seed=10, std=0.5)
    w.q = (w.q.astype(np.float32) * 8).astype(np.float16)
    _check_small(pa, w, [512])


# ---------------------------------------------------------------------------
# edge cases and contract violations (NaN rows, skipped writes)
# ---------------------------------------------------------------------------

def test_zero_context_gives_zero_rows(pa):
    w = wl.make_custom([5, 40, 9], n_q_heads=4, n_kv_heads=2, d_head=64,
                       block_size=16, dtype="f32", seed=11)
    d = DeviceBatch(w)
    run_write(pa, d)
    d.context_lens[1] = 0
    for out in (run_decode(pa, d), run_partitioned(pa, d, 16)[0]):
        o = from_dev(out)
        assert (o[1] == 0).all() and np.isfinite(o).all()


def test_contract_violations_give_nan_rows(pa):
    w = wl.make_custom([50, 60, 70, 80], n_q_heads=8, n_kv_heads=2,
                       d_head=128, block_size=16, dtype="bf16", seed=12)
    d = DeviceBatch(w)
    run_write(pa, d)
    good = as_f64(run_decode(pa, d))
    d.block_table[1, 2] = w.n_blocks          # block id out of range
    d.block_table[2, 0] = -5                  # negative block id
    d.context_lens[3] = w.max_blocks * 16 + 1  # longer than the table
    for out in (as_f64(run_decode(pa, d)), as_f64(run_partitioned(pa, d)[0])):
        assert np.isnan(out[1:]).all()
        assert np.array_equal(out[0], good[0])


def test_too_small_workspace_gives_nan(pa):
    w = wl.make_custom([100, 1000], n_q_heads=4, n_kv_heads=2, d_head=64,
                       block_size=16, dtype="f16", seed=13)
    d = DeviceBatch(w)
    run_write(pa, d)
    out, _ = run_partitioned(pa, d, partition_size=64, max_partitions=4)
    o = as_f64(out)
    assert np.isfinite(o[0]).all() and np.isnan(o[1]).all()


def test_cache_write_skips_negative_and_out_of_range_slots(pa):
    w = wl.make_custom([20, 30, 40, 50], n_q_heads=4, n_kv_heads=2,
                       d_head=128, block_size=16, dtype="f16", seed=14)
    slots = w.slot_mapping.copy()
    slots[1] = -1
    slots[2] = w.n_blocks * 16 + 3            # past the pool: skipped
    w.slot_mapping = slots
    d = DeviceBatch(w)
    run_write(pa, d)
    s_ok = slots.copy()
    s_ok[2] = -1
    k_ref, v_ref = oracle.oracle_cache_write(w.k_pool, w.v_pool, w.key_new,
                                             w.value_new, s_ok, 16)
    assert from_dev(d.k_pool).tobytes() == k_ref.tobytes()
    assert from_dev(d.v_pool).tobytes() == v_ref.tobytes()


def test_full_pool_fill_by_cache_write(pa):
    """Writing every cached token through pa_cache_write (one call per
    position index) rebuilds the generator's pool exactly."""
    w = wl.make_custom([33, 17, 64], n_q_heads=4, n_kv_heads=2, d_head=64,
                       block_size=16, dtype="bf16", seed=15, poison=True)
    k_ref, v_ref = oracle_pools_after_write(w)
    target_k = torch.full_like(to_dev(w.k_pool, "bf16"), float("nan"))
    target_v = torch.full_like(target_k, float("nan"))
    BS = 16
    for t in range(int(w.context_lens.max())):
        keys, vals, slots = [], [], []
        for b in range(3):
            if t < w.context_lens[b]:
                blk = w.block_table[b, t // BS]
                keys.append(k_ref[blk, :, t % BS])
                vals.append(v_ref[blk, :, t % BS])
                slots.append(blk * BS + t % BS)
        pa.pa_cache_write(to_dev(np.stack(keys), "bf16"),
                          to_dev(np.stack(vals), "bf16"), target_k, target_v,
                          to_dev(np.array(slots, dtype=np.int32)))
    sync()
    assert from_dev(target_k).tobytes() == k_ref.tobytes()
    assert from_dev(target_v).tobytes() == v_ref.tobytes()


def test_empty_batch_is_a_noop(pa):
    z = torch.empty((0, 4, 64), dtype=torch.float32, device="cuda")
    kp = torch.zeros((2, 2, 16, 64), dtype=torch.float32, device="cuda")
    tbl = torch.zeros((0, 1), dtype=torch.int32, device="cuda")
    cl = torch.zeros((0,), dtype=torch.int32, device="cuda")
    pa.pa_decode(z, z, kp, kp, tbl, cl, scale=0.1)
    pa.pa_cache_write(torch.empty((0, 2, 64), device="cuda"),
                      torch.empty((0, 2, 64), device="cuda"), kp, kp,
                      torch.empty((0,), dtype=torch.int32, device="cuda"))
    sync()
    assert (kp == 0).all()
