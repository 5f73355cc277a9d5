"""pa_copy_blocks (copy-on-write block copy) vs the oracle, through the C ABI
(needs an MI355X).  Bit for bit over the whole of both pools, for every
element type, head width and block size, with rows that name blocks outside
the pool, and at the size of the LLaMA-3-8B batch's pool."""

import numpy as np
import pytest
import torch

import oracle
from helpers import from_dev, note, to_dev
from paged_kv_cache_222_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_222_amd as pa
    pa.load()
    return pa


def _random_pools(rng, shape, dtype):
    """Pools of arbitrary bit patterns (NaNs and infinities included)."""
    if dtype == "f32":
        bits = rng.integers(0, 2**32, shape, dtype=np.uint64).astype(np.uint32)
        return bits.view(np.float32), None
    bits = rng.integers(0, 2**16, shape).astype(np.uint16)
    return (bits if dtype == "bf16" else bits.view(np.float16)), None


def _run(pa, k0, v0, pairs, dtype, name):
    k, v = to_dev(k0, dtype), to_dev(v0, dtype)
    p = torch.from_numpy(pairs).to("cuda")
    note(f"pa_copy_blocks {name} pool {k0.shape} pairs {len(pairs)}")
    pa.pa_copy_blocks(k, v, p)
    torch.cuda.synchronize()
    return from_dev(k), from_dev(v)


def _bits(a):
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint16)


@pytest.mark.parametrize("dtype,H,BS,D", [
    ("bf16", 8, 16, 128), ("f16", 2, 8, 64), ("f32", 3, 32, 64),
    ("bf16", 1, 64, 128), ("f16", 4, 16, 128)])
def test_copy_blocks_bit_exact(pa, dtype, H, BS, D):
    rng = np.random.default_rng(H * 1000 + BS * 10 + D)
    nb = 96
    k0, _ = _random_pools(rng, (nb, H, BS, D), dtype)
    v0, _ = _random_pools(rng, (nb, H, BS, D), dtype)
    pairs = wl.make_copy_pairs(nb, 40, seed=D + BS, invalid=6)
    k, v = _run(pa, k0, v0, pairs, dtype, f"{dtype} H{H} BS{BS} D{D}")
    kr, vr = oracle.oracle_copy_blocks(k0, v0, pairs)
    assert np.array_equal(_bits(k), _bits(kr))
    assert np.array_equal(_bits(v), _bits(vr))


def test_copy_blocks_no_pairs_is_a_noop(pa):
    rng = np.random.default_rng(3)
    k0, _ = _random_pools(rng, (8, 2, 16, 64), "bf16")
    v0, _ = _random_pools(rng, (8, 2, 16, 64), "bf16")
    k, v = _run(pa, k0, v0, np.zeros((0, 2), np.int32), "bf16", "empty")
    assert np.array_equal(k, k0) and np.array_equal(v, v0)


def test_copy_blocks_llama3_pool(pa):
    """The LLaMA-3-8B batch's pool (13,629 blocks in use at seed 0) plus
    4,096 free blocks, 4,096 copies into the free blocks, as the benchmark
    runs it; the whole pool compared."""
    w = wl.make_workload("llama3-8b", seed=0)
    c = w.cfg
    extra = 4096
    pad = np.zeros((extra,) + w.k_pool.shape[1:], w.k_pool.dtype)
    k0 = np.concatenate([w.k_pool, pad])
    v0 = np.concatenate([w.v_pool, pad])
    n_used = w.k_pool.shape[0]
    rng = np.random.default_rng(11)
    src = rng.integers(0, n_used, extra).astype(np.int32)
    dst = (n_used + rng.permutation(extra)).astype(np.int32)
    pairs = np.ascontiguousarray(np.stack([src, dst], axis=1))
    k, v = _run(pa, k0, v0, pairs, c.dtype, "llama3-8b pool")
    kr, vr = oracle.oracle_copy_blocks(k0, v0, pairs)
    assert np.array_equal(_bits(k), _bits(kr))
    assert np.array_equal(_bits(v), _bits(vr))
