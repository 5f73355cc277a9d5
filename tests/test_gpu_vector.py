"""pa_decode_partitioned_vector (the vector-ALU kernel on 16-bit caches) vs
the fp64 oracle, through the C ABI (needs an MI355X).

The entry point exists to time the vector-ALU and matrix-core engines on the
same batch, so it is held to the same bar as the matrix-core path: every
output element within the stated bound, on ragged small batches of every
16-bit type, head width and group size, and on the full LLaMA-3 batch.
"""

import numpy as np
import pytest
import torch

from helpers import (TOL, DeviceBatch, as_f64, from_dev, full_batch, note,
                     oracle_out, oracle_pools_after_write, out_bound)
from paged_kv_cache_222_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_222_amd as pa
    pa.load()
    return pa


def run_vector(pa, d, P, pm=None, name=""):
    pm = pm or max(1, -(-int(d.w.context_lens.max()) // P))
    B, Hq, D = d.q.shape
    ws = pa.partition_workspace(B, Hq, D, pm)
    for t in ws:
        t.fill_(float("nan"))
    note(f"pa_decode_partitioned_vector+pa_reduce {name} P={P} PMAX={pm}")
    pa.pa_decode_partitioned(*ws, d.q, d.k_pool, d.v_pool, d.block_table,
                             d.context_lens, partition_size=P, scale=d.scale,
                             vector=True)
    out = d.empty_out()
    pa.pa_reduce(out, *ws, d.context_lens, partition_size=P)
    torch.cuda.synchronize()
    return out


RAGGED = [1, 2, 7, 8, 9, 15, 16, 17, 33, 64, 100, 129, 257, 513, 1000]
CASES = [(dt, D, BS, G) for dt in ("f16", "bf16") for D in (64, 128)
         for BS, G in ((16, 1), (16, 4), (32, 8), (16, 12))]


@pytest.mark.parametrize("dt,D,BS,G", CASES,
                         ids=[f"{a}-d{b}-bs{c}-g{g}" for a, b, c, g in CASES])
def test_small_batches(pa, dt, D, BS, G):
    n_kv = 2
    w = wl.make_custom(RAGGED, n_q_heads=n_kv * G, n_kv_heads=n_kv, d_head=D,
                       block_size=BS, dtype=dt, seed=3 * G + D + BS,
                       pool_blocks=None)
    d = DeviceBatch(w)
    pa.pa_cache_write(d.key_new, d.value_new, d.k_pool, d.v_pool,
                      d.slot_mapping)
    torch.cuda.synchronize()
    k_ref, v_ref = oracle_pools_after_write(w)
    assert from_dev(d.k_pool).tobytes() == k_ref.tobytes()
    ref = oracle_out(w, k_ref, v_ref)
    bound = out_bound(ref, dt)
    for P in sorted({BS, 64, 512}):
        got = as_f64(run_vector(pa, d, P, name=f"{dt} d{D} bs{BS} g{G}"))
        err = np.abs(got - ref)
        assert (err <= bound).all(), (P, float(err.max()))


def test_zero_context_and_contract_violations(pa):
    w = wl.make_custom([50, 60, 70, 80, 90], n_q_heads=8, n_kv_heads=2,
                       d_head=128, block_size=16, dtype="bf16", seed=12)
    d = DeviceBatch(w)
    pa.pa_cache_write(d.key_new, d.value_new, d.k_pool, d.v_pool,
                      d.slot_mapping)
    torch.cuda.synchronize()
    good = as_f64(run_vector(pa, d, 64))
    d.block_table[1, 2] = w.n_blocks          # block id out of range
    d.block_table[2, 0] = -5                  # negative block id
    d.context_lens[3] = w.max_blocks * 16 + 1  # longer than the table
    d.context_lens[4] = 0                      # nothing cached
    out = as_f64(run_vector(pa, d, 64))
    assert np.isnan(out[1:4]).all()
    assert (out[4] == 0).all()
    assert np.array_equal(out[0], good[0])


def test_full_llama3_batch(pa):
    """The batch the two engines are timed on: every row within TOL."""
    w, k_ref, v_ref, ref = full_batch("llama3-8b")
    d = DeviceBatch(w)
    pa.pa_cache_write(d.key_new, d.value_new, d.k_pool, d.v_pool,
                      d.slot_mapping)
    torch.cuda.synchronize()
    got = as_f64(run_vector(pa, d, w.cfg.partition_size, name="llama3-8b"))
    err = float(np.max(np.abs(got - ref)))
    print(f"llama3-8b vector-ALU partitioned: max err {err:.3g}")
    assert err <= TOL["bf16"]
