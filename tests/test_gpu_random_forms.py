"""Every partitioned form of the decode step on seeded random shapes, against
the fp64 oracle through the C ABI (needs an MI355X): pa_decode_step,
pa_decode_shared_prefix (with a random prefix, sometimes none),
pa_decode_split (fp16/bf16) and pa_cache_write + pa_decode_partitioned, each
followed by pa_reduce.  Shapes draw the element type, head width, block
size, KV heads, group size (1-16), batch (1-39, and 200-299), partition size
and prefix length; every output element within the stated bound and the
pools bit-exact after the write."""

import numpy as np
import pytest
import torch

from helpers import (DeviceBatch, as_f64, from_dev, note, oracle_out,
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


def _shape(seed):
    rng = np.random.default_rng(seed)
    dtype = str(rng.choice(["bf16", "f16", "f32"], p=[0.45, 0.35, 0.2]))
    D = int(rng.choice([64, 128]))
    BS = int(rng.choice([8, 16, 32, 64]))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
    B = int(rng.integers(1, 40)) if rng.random() < 0.8 else int(rng.integers(200, 300))
    P = BS * int(rng.integers(1, 9)) * (2 if BS < 32 else 1) * (1 if rng.random() < 0.8 else 8)
    plen = int(rng.choice([0, P, 2 * P, P + BS, 3 * P]))
    ctx = [plen + 1 + int(x) for x in rng.integers(0, 1500 if B < 100 else 300, B)]
    return dtype, D, BS, Hkv, G, B, P, plen, ctx


@pytest.mark.parametrize("seed", range(40))
def test_random_shape_every_form(pa, seed):
    dtype, D, BS, Hkv, G, B, P, plen, ctx = _shape(seed)
    w = wl.make_custom(ctx, n_q_heads=Hkv * G, n_kv_heads=Hkv, d_head=D,
                       block_size=BS, dtype=dtype, seed=5000 + seed,
                       prefix_len=plen)
    k_ref, v_ref = oracle_pools_after_write(w)
    ref = oracle_out(w, k_ref, v_ref)
    bound = out_bound(ref, dtype)
    pm = max(1, -(-max(ctx) // P))
    forms = ["step", "prefix", "partitioned"] + (["split"] if dtype != "f32" else [])
    for form in forms:
        d = DeviceBatch(w)
        note(f"seed {seed} {form}: {dtype} D{D} BS{BS} Hkv{Hkv} G{G} B{B} "
             f"P{P} prefix{plen}")
        if form == "partitioned":
            pa.pa_cache_write(d.key_new, d.value_new, d.k_pool, d.v_pool,
                              d.slot_mapping)
        slots = max(2, min(16, pm + 2)) if form == "split" else pm
        ws = pa.partition_workspace(B, Hkv * G, D, slots)
        for t in ws:
            t.fill_(float("nan"))
        if form == "step":
            pa.pa_decode_step(*ws, d.key_new, d.value_new, d.q, d.k_pool,
                              d.v_pool, d.block_table, d.context_lens,
                              partition_size=P, scale=d.scale)
        elif form == "prefix":
            pa.pa_decode_shared_prefix(
                *ws, d.q, d.k_pool, d.v_pool, d.block_table, d.context_lens,
                partition_size=P, prefix_len=plen, scale=d.scale,
                key_new=d.key_new, value_new=d.value_new)
        elif form == "split":
            pa.pa_decode_split(*ws, d.q, d.k_pool, d.v_pool, d.block_table,
                               d.context_lens, scale=d.scale,
                               key_new=d.key_new, value_new=d.value_new)
        else:
            pa.pa_decode_partitioned(*ws, d.q, d.k_pool, d.v_pool,
                                     d.block_table, d.context_lens,
                                     partition_size=P, scale=d.scale)
        out = d.empty_out()
        pa.pa_reduce(out, *ws, d.context_lens,
                     partition_size=0 if form == "split" else P)
        torch.cuda.synchronize()
        assert from_dev(d.k_pool).tobytes() == k_ref.tobytes(), form
        assert from_dev(d.v_pool).tobytes() == v_ref.tobytes(), form
        err = np.abs(as_f64(out) - ref)
        assert (err <= bound).all(), (form, float(np.nanmax(err)))
