"""pa_decode_step (the cache write folded into the partitioned attention)
against pa_cache_write followed by pa_decode_partitioned, through the C ABI
(needs an MI355X): the pools, the partition workspace and the reduced output
must be bit-identical, and the output within the stated tolerance of the
fp64 oracle.  Covers every element type, both head widths, every block
size, a new token that opens a partition or a block, a one-token sequence,
and the full LLaMA-3-8B batch."""

import numpy as np
import pytest
import torch

from helpers import (TOL, DeviceBatch, as_f64, from_dev, note, oracle_out,
                     oracle_pools_after_write, out_bound)
from paged_kv_cache_222_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_222_amd as pa
    pa.load()
    return pa


def _bits(t):
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy()
    return t.view(torch.int32).numpy()


def _both(pa, w, P, name):
    """(fused, separate) results: (k_pool, v_pool, workspace, out)."""
    res = []
    pm = max(1, -(-int(w.context_lens.max()) // P))
    for fused in (True, False):
        d = DeviceBatch(w)
        B, Hq, D = d.q.shape
        ws = pa.partition_workspace(B, Hq, D, pm)
        for t in ws:
            t.fill_(float("nan"))
        if fused:
            note(f"pa_decode_step {name} P={P}")
            pa.pa_decode_step(*ws, d.key_new, d.value_new, d.q, d.k_pool,
                              d.v_pool, d.block_table, d.context_lens,
                              partition_size=P, scale=d.scale)
        else:
            note(f"pa_cache_write+pa_decode_partitioned {name} P={P}")
            pa.pa_cache_write(d.key_new, d.value_new, d.k_pool, d.v_pool,
                              d.slot_mapping)
            pa.pa_decode_partitioned(*ws, d.q, d.k_pool, d.v_pool,
                                     d.block_table, d.context_lens,
                                     partition_size=P, scale=d.scale)
        out = d.empty_out()
        pa.pa_reduce(out, *ws, d.context_lens, partition_size=P)
        torch.cuda.synchronize()
        res.append((d.k_pool, d.v_pool, ws, out))
    return res


def _check_identical(fused, sep):
    for a, b in zip(fused[:2], sep[:2]):
        assert np.array_equal(_bits(a), _bits(b))
    for a, b in zip(fused[2], sep[2]):
        assert np.array_equal(_bits(a), _bits(b))
    assert np.array_equal(_bits(fused[3]), _bits(sep[3]))


CASES = [  # dtype, D, BS, Hkv, G, P
    ("bf16", 128, 16, 2, 4, 64), ("f16", 64, 8, 1, 6, 32),
    ("bf16", 128, 32, 4, 1, 128), ("f32", 64, 16, 2, 2, 64),
    ("f16", 128, 64, 1, 8, 128), ("bf16", 64, 16, 3, 5, 16)]


@pytest.mark.parametrize("dtype,D,BS,Hkv,G,P", CASES)
def test_step_equals_write_then_decode(pa, dtype, D, BS, Hkv, G, P):
    # lengths where the new token is a partition's or a block's first
    # position, a one-token sequence, and ragged others
    ctx = [1, 2, P + 1, 2 * P + 1, BS + 1, 17, 100, 3 * P, 5 * P - 3]
    w = wl.make_custom(ctx, n_q_heads=Hkv * G, n_kv_heads=Hkv, d_head=D,
                       block_size=BS, dtype=dtype, seed=D + G + P)
    fused, sep = _both(pa, w, P, f"{dtype} D{D} BS{BS} G{G}")
    _check_identical(fused, sep)
    k_ref, v_ref = oracle_pools_after_write(w)
    assert from_dev(fused[0]).tobytes() == k_ref.tobytes()
    assert from_dev(fused[1]).tobytes() == v_ref.tobytes()
    ref = oracle_out(w, k_ref, v_ref)
    err = np.abs(as_f64(fused[3]) - ref)
    assert (err <= out_bound(ref, dtype)).all()


def test_step_llama3_full_batch(pa):
    w = wl.make_workload("llama3-8b", seed=0)
    fused, sep = _both(pa, w, w.cfg.partition_size, "llama3-8b")
    _check_identical(fused, sep)


@pytest.mark.parametrize("dtype,B", [("bf16", 9), ("f16", 1030), ("f32", 9)])
def test_undersized_workspace_still_writes(pa, dtype, B):
    """A workspace with fewer partitions than some sequence needs: those
    rows come out NaN (pa_reduce), the others match the oracle, and the new
    token of every sequence is still in the pools, bit for bit as
    pa_cache_write puts it.  B = 1030 runs the launch without the in-kernel
    plan (one work group per partition row); fp32 runs its own write."""
    P = 32
    rng = np.random.default_rng(31 + B)
    ctx = [int(c) for c in rng.integers(1, 4 * P, size=B)]
    ctx[0], ctx[1] = 5 * P, 3 * P + 1     # need 5 and 4 partitions
    pm = 3
    w = wl.make_custom(ctx, n_q_heads=8, n_kv_heads=2, d_head=64,
                       block_size=16, dtype=dtype, seed=40 + B)
    d = DeviceBatch(w)
    Bq, Hq, D = d.q.shape
    ws = pa.partition_workspace(Bq, Hq, D, pm)
    note(f"pa_decode_step {dtype} B={B} P={P} PMAX={pm} (undersized)")
    pa.pa_decode_step(*ws, d.key_new, d.value_new, d.q, d.k_pool, d.v_pool,
                      d.block_table, d.context_lens, partition_size=P,
                      scale=d.scale)
    out = d.empty_out()
    pa.pa_reduce(out, *ws, d.context_lens, partition_size=P)
    torch.cuda.synchronize()
    k_ref, v_ref = oracle_pools_after_write(w)
    assert from_dev(d.k_pool).tobytes() == k_ref.tobytes()
    assert from_dev(d.v_pool).tobytes() == v_ref.tobytes()
    got = as_f64(out)
    over = np.array([-(-c // P) > pm for c in ctx])
    assert over[0] and over[1]
    assert np.isnan(got[over]).all()
    ref = oracle_out(w, k_ref, v_ref)
    err = np.abs(got[~over] - ref[~over])
    assert (err <= out_bound(ref[~over], dtype)).all()
