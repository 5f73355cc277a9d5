"""pa_decode_step_noalloc through the C ABI (needs an MI355X): the decode
step with its partition workspace in the library's fixed scratch buffer.
Its pools and output must equal those of pa_decode_step + pa_reduce (the
entry point it varies, workspace from caller memory) bit for bit, on two
calls in a row -- the second on a smaller batch, so contents the first call
left in the buffer must not leak -- and it must refuse, with nothing
enqueued, a workspace beyond the buffer's 32 MiB."""

import numpy as np
import pytest
import torch

from helpers import DeviceBatch, from_dev, note, oracle_out, \
    oracle_pools_after_write, out_bound, as_f64
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


def _reference(pa, w, P):
    """pa_decode_step + pa_reduce with caller-allocated workspace sized as
    the no-allocation call sizes its own: ceil(max_blocks * bs / P)."""
    d = DeviceBatch(w)
    B, Hq, D = d.q.shape
    pm = -(-w.max_blocks * w.cfg.block_size // P)
    ws = pa.partition_workspace(B, Hq, D, pm)
    note(f"reference pa_decode_step+pa_reduce B={B} P={P} PMAX={pm}")
    pa.pa_decode_step(*ws, d.key_new, d.value_new, d.q, d.k_pool, d.v_pool,
                      d.block_table, d.context_lens, partition_size=P,
                      scale=d.scale)
    out = d.empty_out()
    pa.pa_reduce(out, *ws, d.context_lens, partition_size=P)
    torch.cuda.synchronize()
    return d, out


def _noalloc(pa, w, P):
    d = DeviceBatch(w)
    out = d.empty_out()
    note(f"pa_decode_step_noalloc B={d.q.shape[0]} P={P}")
    pa.pa_decode_step_noalloc(out, d.key_new, d.value_new, d.q, d.k_pool,
                              d.v_pool, d.block_table, d.context_lens,
                              partition_size=P, scale=d.scale)
    torch.cuda.synchronize()
    return d, out


def _same(a, b):
    (da, oa), (db, ob) = a, b
    assert np.array_equal(_bits(oa), _bits(ob))
    assert np.array_equal(_bits(da.k_pool), _bits(db.k_pool))
    assert np.array_equal(_bits(da.v_pool), _bits(db.v_pool))


@pytest.mark.parametrize("dtype,D,G", [("bf16", 128, 4), ("f16", 64, 6),
                                       ("f32", 64, 2)])
def test_two_calls_in_a_row_match_the_step(pa, dtype, D, G):
    P = 64
    rng = np.random.default_rng(70 + D + G)
    big = [int(c) for c in rng.integers(1, 700, size=37)]
    big[0] = 700
    small = [int(c) for c in rng.integers(1, 150, size=5)]
    for ctx, seed in ((big, 1), (small, 2)):      # the second one smaller
        w = wl.make_custom(ctx, n_q_heads=2 * G, n_kv_heads=2, d_head=D,
                           block_size=16, dtype=dtype, seed=seed + D)
        got = _noalloc(pa, w, P)
        _same(got, _reference(pa, w, P))
        k_ref, v_ref = oracle_pools_after_write(w)
        assert from_dev(got[0].k_pool).tobytes() == k_ref.tobytes()
        ref = oracle_out(w, k_ref, v_ref)
        err = np.abs(as_f64(got[1]) - ref)
        assert (err <= out_bound(ref, dtype)).all()


def test_llama3_batch_matches_the_step(pa):
    w = wl.make_workload("llama3-8b", seed=0)
    P = w.cfg.partition_size
    _same(_noalloc(pa, w, P), _reference(pa, w, P))


def test_workspace_beyond_the_buffer_is_refused(pa):
    # 256 sequences x 32 heads x 16 partitions x 130 floats = 68 MB > 32 MiB
    ctx = [100] * 256
    w = wl.make_custom(ctx, n_q_heads=32, n_kv_heads=8, d_head=128,
                       block_size=16, dtype="bf16", seed=3, max_context=8192)
    d = DeviceBatch(w)
    k0 = from_dev(d.k_pool).tobytes()
    out = d.empty_out()
    with pytest.raises(pa.PaError) as e:
        pa.pa_decode_step_noalloc(out, d.key_new, d.value_new, d.q, d.k_pool,
                                  d.v_pool, d.block_table, d.context_lens,
                                  partition_size=512, scale=d.scale)
    assert e.value.status == -9
    torch.cuda.synchronize()
    assert from_dev(d.k_pool).tobytes() == k0          # nothing ran
    assert np.isnan(as_f64(out)).all()
