"""bench.py's reporting helpers, on the CPU: the algorithmic bytes of a
launch (the sum of the per-sequence terms, written out independently here),
the number of resident input copies, and the lookup of stored HBM counters
(matched on form, partition and block size; null once the kernel sources
change)."""

import os
import re
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import pytest  # noqa: E402

import bench  # noqa: E402
from paged_kv_cache_222_amd import workloads as wl  # noqa: E402


@pytest.fixture(scope="module")
def llama3():
    return wl.make_workload("llama3-8b", seed=0)


def test_algorithmic_bytes_of_the_llama3_batch(llama3):
    """Per sequence-step: K and V rows of every KV head, the queries, the
    used table entries and the context length.  Seed 0: sum(ctx) = 217,087."""
    w = llama3
    c = w.cfg
    ctx = w.context_lens.astype(np.int64)
    want = 0
    for n in ctx:
        want += 2 * int(n) * c.n_kv_heads * c.d_head * 2          # K and V
        want += c.n_q_heads * c.d_head * 2                       # q
        want += 4 * -(-int(n) // c.block_size)                   # table
        want += 4                                                 # length
    assert int(ctx.sum()) == 217087
    assert bench.algorithmic_bytes(w) == want == 890291956


def test_resident_copies_leave_the_last_level_cache(llama3):
    class A:
        copies = None
    for name, want in (("llama3-8b", 3), ("qwen2.5-1.5b", 8), ("tiny", 16)):
        w = llama3 if name == "llama3-8b" else wl.make_workload(name, seed=0)
        n = bench.n_copies(A, w)
        assert n == want, name
        per = w.kv_bytes_unique() if w.cfg.prefix_len else w.kv_bytes_logical()
        # at least 1 GiB of other K/V reads between two uses of a copy,
        # unless capped (a batch too small to leave the cache)
        assert n == 16 or (n - 1) * per >= (1 << 30), name
    A.copies = 5
    assert bench.n_copies(A, wl.make_workload("tiny", seed=0)) == 5


def test_traffic_lookup_matches_form_and_sources(monkeypatch):
    # the committed LLaMA-3 counters are for the fused form at P 3072, BS 16
    got = bench.measured_traffic("llama3-8b", "fused", 3072, 16)
    if got is not None:       # the sources match the stored hash
        assert 890_000_000 < got < 910_000_000
    assert bench.measured_traffic("llama3-8b", "split", 3072, 16) is None
    assert bench.measured_traffic("llama3-8b", "fused", 2048, 16) is None
    assert bench.measured_traffic("llama3-8b", "fused", 3072, 32) is None
    assert bench.measured_traffic("no-such-batch", "fused", 3072, 16) is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.measured_traffic("llama3-8b", "fused", 3072, 16) is None


@pytest.mark.parametrize("name,form,P", [
    ("llama3-8b", "fused", 3072), ("qwen2.5-1.5b", "fused", 1536),
    ("llama2-7b", "partitioned", 4096), ("shared-prefix", "prefix", 512)])
def test_every_headline_form_has_counters(name, form, P):
    """Each batch's reported form has HBM counters under profiles/ for its
    partition size, so the bench line can carry them; when the kernel
    sources still match the ones they were taken on, the traffic is within
    a few percent of the algorithmic bytes stated beside it."""
    if name in bench.HEADLINE_FORM:
        assert bench.HEADLINE_FORM[name] == form
    found = None
    for fname in os.listdir(os.path.join(ROOT, "profiles")):
        if not fname.endswith("_hbm_counters.txt") or f"_{name}_" not in fname:
            continue
        kv = {}
        text = open(os.path.join(ROOT, "profiles", fname)).read()
        for line in text.splitlines():
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if kv.get("variant") == form and kv.get("partition_size") == str(P):
            m = re.search(r"Algorithmic bytes per launch \(bench.py's figure for this "
                          r"launch\) are (\d+)", " ".join(text.split()))
            found = (kv, int(m.group(1)) if m else None)
    assert found is not None, f"no counters for {name} {form} P{P}"
    kv, alg = found
    got = bench.measured_traffic(name, form, P, int(kv["block_size"]))
    if kv["source_sha256_16"] == bench.kernel_source_hash():
        assert got is not None and alg is not None
        assert 1.0 <= got / alg < 1.03, (name, got / alg)
    else:
        assert got is None
