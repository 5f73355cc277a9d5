"""Throughput of one paged-attention decode step on one MI355X.

A step is the whole hot path over one batch: the cache write of each
sequence's new token, then attention over every sequence's paged cache.
Four forms are timed: "fused" (pa_decode_step -- the write folded into the
partitioned attention -- then pa_reduce), "split" (pa_decode_split: the
context cut into pieces of equal runs of tiles, the write folded in, then
pa_reduce), "partitioned" (pa_cache_write, pa_decode_partitioned,
pa_reduce) and "single" (pa_cache_write, the single-pass pa_decode); the
line reports the batch's headline form (see HEADLINE_FORM), the others'
times beside it (--variant best reports the fastest instead).  A batch
whose rows share a prompt's blocks also times "prefix"
(pa_decode_shared_prefix with the write folded in, then pa_reduce) and
reports that.  "vector" (pa_cache_write, pa_decode_partitioned_vector,
pa_reduce: the partitioned form on the vector-ALU kernel) is timed only
when asked for, to set the two engines side by side.  Inputs are seeded
synthetic batches (see
paged_kv_cache_222_amd/workloads.py); the default is the LLaMA-3-8B-shaped
GQA batch (B=128, 32/8 heads, d128, bf16, log-normal context lengths).
Several copies of the inputs are resident in HBM and the steps rotate over
them, so no step finds the previous step's K/V in the 256 MB last-level
cache.

Prints one JSON line: KV-read GB/s (value), seq-steps/s, fraction of the
8 TB/s HBM peak, the dominant kernel's roofline figures -- its duration from
the timestamps of its own dispatch, recorded in HIP events on the stream it
runs on (pa_time_next_attention) -- the achievable read ceiling measured on
the same device (pa_read_ceiling), and the fp64 CPU oracle timed on a
bounded sample of the same batch.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = ("paged-attn decode KV-read GB/s (% of 8 TB/s HBM peak) and "
          "seq-steps/s")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama3-8b")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--block-size", type=int, default=None)
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--copies", type=int, default=None,
                    help="resident input copies the steps rotate over "
                         "(default: enough that 1 GiB of other K/V reads "
                         "comes between two uses of a copy, at least 3)")
    ap.add_argument("--variant", choices=["all", "best", "fused", "split",
                                          "partitioned", "single", "prefix",
                                          "vector"],
                    default="all",
                    help="all (default): time every form, report the "
                         "batch's headline form (HEADLINE_FORM; the "
                         "shared-prefix step for a batch with a shared "
                         "prefix); best: report the fastest form; "
                         "vector: the partitioned form on the vector-ALU "
                         "kernel (pa_decode_partitioned_vector), timed only "
                         "when asked for")
    ap.add_argument("--slots", type=int, default=None,
                    help="split form: workspace slots per row (default: the "
                         "fewest that let every work group take an even "
                         "share, from the batch's lengths and the device)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the read-ceiling calibration (pa_read_ceiling "
                         "over a 4 GiB buffer) after the decode timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the CPU oracle sample")
    ap.add_argument("--op", choices=["decode", "copy-blocks", "verify",
                                     "prefix-cache", "timeline"],
                    default="decode",
                    help="decode: the decode step (default); copy-blocks: "
                         "the copy-on-write block copy on the LLaMA-3-8B pool; "
                         "verify: a speculative-decoding verify step, "
                         "--queries tokens per sequence; prefix-cache: the "
                         "host-side block hashes and prefix mapping of the "
                         "shared-prefix batch (no GPU); timeline: per-work-"
                         "group timeline of the attention kernel (a library "
                         "built with -DPA_TIMELINE, named by PA_LIBRARY)")
    ap.add_argument("--queries", type=int, default=4,
                    help="verify: query tokens per sequence")
    ap.add_argument("--pairs", type=int, default=4096,
                    help="copy-blocks: block pairs per call")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB "
                         "five times and exit: the known-size kernel that "
                         "scales the HBM byte counters")
    return ap.parse_args()


def algorithmic_bytes(w):
    """Bytes the attention kernel must move per launch (its roofline unit is
    one sequence-step): every cached K/V row of every KV head, the queries,
    the used block-table entries and the context lengths."""
    c = w.cfg
    nb = {"f32": 4, "f16": 2, "bf16": 2}[c.dtype]
    kv = w.kv_bytes_logical()
    q = c.batch * c.n_q_heads * c.d_head * nb
    tbl = 4 * int((-(-w.context_lens.astype(np.int64) // c.block_size)).sum())
    return kv + q + tbl + 4 * c.batch


# The form each batch's line reports by default (--variant all): the fastest
# form measured on MI355X for that batch (a batch with a shared prefix
# reports "prefix").
HEADLINE_FORM = {"llama3-8b": "fused", "qwen2.5-1.5b": "fused",
                 "llama2-7b": "partitioned", "tiny": "fused"}

# sources whose change invalidates the HBM byte counts stored under profiles/
KERNEL_SOURCES = ["pa_attention_mfma.h", "pa_attention_mfma.hip",
                  "pa_attention.h", "pa_attention_vector.hip",
                  "pa_launch.h", "pa_device.h", "pa_api.hip"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_222_amd", "csrc", f),
                  "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name, variant, P, block_size):
    """HBM bytes per attention launch from a counter summary stored under
    profiles/ (FETCH_SIZE + WRITE_SIZE, each scaled by the copy-kernel
    factor) for this workload, form, partition and block size, or None when
    there is none or the kernel sources changed since it was taken."""
    kernel = "attention_vector" if variant == "vector" else "attention_mfma"
    for fname in (f"{kernel}_{name}_P{P}_hbm_counters.txt",
                  f"{kernel}_{name}_hbm_counters.txt"):
        path = os.path.join(ROOT, "profiles", fname)
        if not os.path.exists(path):
            continue
        kv = {}
        with open(path) as fh:
            for line in fh:
                if ":" in line and not line.startswith((" ", "#", "\t")):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if (kv.get("source_sha256_16") == kernel_source_hash()
                and kv.get("variant") == variant
                and kv.get("partition_size") == str(P)
                and kv.get("block_size", "16") == str(block_size)):
            try:
                return int(kv["traffic_bytes_per_launch"])
            except (KeyError, ValueError):
                return None
    return None


def n_copies(args, w):
    """Resident input copies the steps rotate over: --copies, else enough
    that at least 1 GiB of other K/V reads (four times the 256 MB last-level
    cache) falls between two steps on the same copy; 3 to 16 (a batch too
    small for 16 copies to leave the cache is cache-resident anyway)."""
    if args.copies:
        return args.copies
    per_step = w.kv_bytes_unique() if w.cfg.prefix_len else w.kv_bytes_logical()
    return min(16, max(3, 1 + -(-(1 << 30) // max(1, per_step))))


def split_slots(w, torch):
    """Workspace slots for pa_decode_split: the fewest that let every work
    group take an even share of the tiles.  A column (KV head and chunk of
    16 query columns) has 2 * CUs / columns work groups (two per CU fit);
    its even share is R = ceil(tiles / work groups) tiles, and a sequence of
    T tiles is cut into at most ceil(T / R) + 1 pieces."""
    c = w.cfg
    cols = c.n_kv_heads * -(-c.gqa_group // 16)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wg = max(1, (2 * cus) // cols)
    tiles = -(-w.context_lens.astype(np.int64) // 16)
    share = -(-int(tiles.sum()) // wg)
    return int(max(2, min(16, -(-int(tiles.max()) // share) + 1)))


def measure_read_ceiling(torch, pa, gib=4, reps=10, batch_tiles=0):
    """The device's achievable HBM read rate for the attention kernels'
    access pattern: pa_read_ceiling over a ``gib`` GiB buffer, in address
    order and as a gather of its 4 KiB tiles in a random order (median of
    ``reps`` launches, each timed by its own dispatch's timestamps through
    pa_time_next_attention, on torch's current stream, the stream the
    launches go to).  With ``batch_tiles``, also the gather of only that many
    tiles -- as many bytes as one decode step reads -- whose rate includes
    the start and end of a launch of that size; its launches rotate over
    disjoint sets of tiles (at least 3, as the decode steps rotate over input
    copies) so that no launch finds its tiles in the last-level cache."""
    nbytes = gib << 30
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    n_tiles = nbytes // 4096
    gen = torch.Generator(device="cpu").manual_seed(0)
    order = torch.randperm(n_tiles, generator=gen).to(torch.int32).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = {"buffer_bytes": nbytes, "tile_bytes": 4096}
    legs = [("stream", [{}]), ("tile_gather", [{"tile_order": order}])]
    if batch_tiles:
        nb = int(batch_tiles)
        sets = min(8, n_tiles // nb)
        if sets >= 3:
            legs.append(("batch_size_tile_gather",
                         [{"tile_order": order[k * nb:(k + 1) * nb]}
                          for k in range(sets)]))
            res["batch_size_tile_sets"] = sets
    for name, kws in legs:
        for kw in kws[:2]:
            pa.pa_read_ceiling(buf, sink, **kw)
        torch.cuda.synchronize()
        ts = []
        for r in range(reps):
            e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            pa.pa_time_next_attention(e0, e1)
            pa.pa_read_ceiling(buf, sink, **kws[(r + 2) % len(kws)])
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        moved = (kws[0]["tile_order"].numel() * 4096
                 if name == "batch_size_tile_gather" else nbytes)
        res[f"{name}_GBs"] = round(moved / (ms * 1e-3) / 1e9, 1)
        if name == "batch_size_tile_gather":
            res[f"{name}_bytes"] = moved
            res[f"{name}_us"] = round(ms * 1e3, 2)
    del buf, order
    torch.cuda.empty_cache()
    return res


def copy_calibration(mib):
    """A plain copy of known size: reads and writes mib MiB per launch."""
    import torch
    n = mib * 2**20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {mib} MiB five times ({mib * 1024} KiB read and written "
        "per launch)")


def bench_copy_blocks(args, torch, pa, wl):
    """pa_copy_blocks on the LLaMA-3-8B pool plus args.pairs free blocks:
    each call copies args.pairs used blocks (K and V, all KV heads) into the
    free ones; three pair lists rotate so that no call finds its sources in
    the last-level cache."""
    w = wl.make_workload("llama3-8b", seed=args.seed)
    c = w.cfg
    n_used = w.k_pool.shape[0]
    n_total = n_used + args.pairs
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[c.dtype]
    shape = (n_total,) + w.k_pool.shape[1:]
    k = torch.empty(shape, dtype=tdt, device="cuda")
    v = torch.empty(shape, dtype=tdt, device="cuda")
    k[:n_used].copy_(torch.from_numpy(w.k_pool.view(np.int16)).view(tdt))
    v[:n_used].copy_(torch.from_numpy(w.v_pool.view(np.int16)).view(tdt))
    lists = []
    for i in range(3):
        rng = np.random.default_rng(1000 + i)
        src = rng.integers(0, n_used, args.pairs)
        dst = n_used + rng.permutation(args.pairs)
        lists.append(torch.from_numpy(np.ascontiguousarray(
            np.stack([src, dst], axis=1).astype(np.int32))).cuda())
    block_bytes = int(np.prod(shape[1:])) * 2
    moved = 2 * 2 * block_bytes * args.pairs        # K and V, read + write
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        pa.pa_copy_blocks(k, v, lists[i % 3])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        pa.pa_copy_blocks(k, v, lists[i % 3])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        pa.pa_copy_blocks(k, v, lists[i % 3])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    ms = wall / args.steps * 1e3
    rec = {
        "metric": "copy-on-write block copy GB/s (bytes read + written)",
        "value": round(moved / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": c.dtype,
        "data": "synthetic",
        "config": {"workload": f"pa_copy_blocks: {args.pairs} blocks of the "
                               f"llama3-8b pool ({n_used} blocks in use, "
                               f"{block_bytes} B per block per pool) into "
                               "free blocks", "pairs": args.pairs,
                   "block_bytes": block_bytes, "seed": args.seed},
        "roofline": {"kernel": "copy_blocks_kernel (pa_copy_blocks)",
                     "bound": "hbm", "achieved": round(moved / (us * 1e-6) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": moved,
                     "avg_launch_us": round(us, 3)},
    }
    if not args.no_cpu_baseline:
        import oracle
        kh = w.k_pool[:min(n_used, 2048)]
        vh = w.v_pool[:min(n_used, 2048)]
        pairs = np.stack([np.arange(0, 512), np.arange(512, 1024)], axis=1)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 10.0):
            oracle.oracle_copy_blocks(kh, vh, pairs)
            reps += 1
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {
            "value": round(reps * 2 * 2 * block_bytes * len(pairs) / dt / 1e9, 4),
            "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} calls of 512 pairs on a 2048-block slice of the "
                      f"pool (numpy copies of whole pools included), {dt:.1f} s"}
    print(json.dumps(rec), flush=True)


def bench_verify(args, torch, pa, wl):
    """The verify pass of speculative decoding on the LLaMA-3-8B batch: the
    cache write of every sequence's last k tokens, then pa_decode_multi
    (k causal query tokens per sequence) and pa_reduce."""
    w = wl.make_workload(args.config, seed=args.seed)
    c = w.cfg
    k = args.queries
    P = args.partition_size or c.partition_size
    pmax = max(1, -(-int(w.context_lens.max()) // P))
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[c.dtype]

    def up(x, dt=None):
        if dt is not None:
            return torch.from_numpy(x.view(np.int16)).view(dt).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    qm = wl.make_multi_queries(w, k, seed=args.seed)
    slots = up(wl.multi_token_slots(w, k))
    rng = np.random.default_rng(args.seed + 7)
    kv_new = wl.encode(rng.standard_normal(
        (c.batch * k, c.n_kv_heads, c.d_head), dtype=np.float32), c.dtype)
    copies = [dict(k=up(w.k_pool, tdt), v=up(w.v_pool, tdt), q=up(qm, tdt),
                   kn=up(kv_new, tdt), vn=up(kv_new, tdt))
              for _ in range(n_copies(args, w))]
    tbl, cl = up(w.block_table), up(w.context_lens)
    B, Hq, D = c.batch, c.n_q_heads, c.d_head
    ws = pa.partition_workspace(B, k * Hq, D, pmax)
    out = torch.empty((B, k, Hq, D), dtype=tdt, device="cuda")
    stream = torch.cuda.current_stream()

    def step(x, ev=None):
        if ev is not None:
            ev[0].record(stream)
        pa.pa_cache_write(x["kn"], x["vn"], x["k"], x["v"], slots)
        if ev is not None:
            ev[1].record(stream)
            pa.pa_time_next_attention(ev[4], ev[5])
        pa.pa_decode_multi(*ws, x["q"], x["k"], x["v"], tbl, cl,
                           partition_size=P, scale=w.scale)
        if ev is not None:
            ev[2].record(stream)
        pa.pa_reduce(out.view(B, k * Hq, D), *ws, cl, partition_size=P)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(copies[i % len(copies)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(copies[i % len(copies)])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)]
           for _ in range(args.steps)]
    for i in range(args.steps):
        step(copies[i % len(copies)], evs[i])
    torch.cuda.synchronize()
    # write, attention call, reduce call, attention kernel (its own
    # timestamps), microseconds
    per = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]),
                     e[2].elapsed_time(e[3]), e[4].elapsed_time(e[5])]
                    for e in evs]) * 1e3
    ms = wall / args.steps * 1e3
    kv = w.kv_bytes_logical()
    attn_us = float(per[:, 3].mean())
    nb = 2
    alg = kv + B * k * Hq * D * nb + 4 * int(
        (-(-w.context_lens.astype(np.int64) // c.block_size)).sum()) + 4 * B
    rec = {
        "metric": "speculative verify step KV-read GB/s (k query tokens per "
                  "sequence, % of 8 TB/s HBM peak)",
        "value": round(kv / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": c.dtype,
        "data": "synthetic",
        "config": {"workload": f"{c.name} verify step: cache write of the "
                               f"last {k} tokens + {k}-token causal attention, "
                               f"one layer: {c.description}",
                   "batch": B, "queries": k, "n_q_heads": Hq,
                   "n_kv_heads": c.n_kv_heads, "d_head": D,
                   "block_size": c.block_size, "partition_size": P,
                   "sum_context": int(w.context_lens.sum()), "seed": args.seed},
        "tokens_per_s": round(B * k / (ms * 1e-3), 1),
        "kernel_us": {"cache_write": round(float(per[:, 0].mean()), 2),
                      "attention": round(attn_us, 2),
                      "reduce": round(float(per[:, 2].mean()), 2)},
        "roofline": {"kernel": "attention_mfma_kernel (pa_decode_multi)",
                     "bound": "hbm",
                     "achieved": round(alg / (attn_us * 1e-6) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(alg / (attn_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"{c.name}_verify{k}",
                                                 "multi", P, c.block_size),
                     "algorithmic_bytes_per_launch": alg,
                     "avg_launch_us": round(attn_us, 3)},
    }
    if not args.no_cpu_baseline:
        import oracle
        k_ref, v_ref = oracle.oracle_cache_write(w.k_pool, w.v_pool,
                                                 w.key_new, w.value_new,
                                                 w.slot_mapping, c.block_size)
        t0 = time.perf_counter()
        done, kvb = 0, 0
        for b in range(B):
            oracle.oracle_decode_multi(qm, k_ref, v_ref, w.block_table,
                                       w.context_lens, w.scale, c.gqa_group,
                                       c.block_size, c.dtype,
                                       rows=[(b, j, h) for j in range(k)
                                             for h in range(Hq)])
            done += 1
            kvb += int(w.context_lens[b]) * c.n_kv_heads * D * 2 * nb
            if time.perf_counter() - t0 > args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {
            "value": round(kvb / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"first {done} of {B} sequences, all {k} tokens and "
                      f"{Hq} heads, fp64 numpy, {dt:.1f} s"}
    print(json.dumps(rec), flush=True)


def bench_timeline(args, torch, pa, wl):
    """Per-work-group timeline of the matrix-core attention kernel, from a
    library built with -DPA_TIMELINE (python -m
    paged_kv_cache_222_amd.build --out=PATH -DPA_TIMELINE; PA_LIBRARY=PATH):
    thread 0 of every work group records s_memrealtime (100 MHz) at its
    start, after the plan and around every item.  Runs --warmup launches,
    then --steps recorded launches of the batch's form (--variant fused,
    split, partitioned or prefix), each on its own resident input copy, and
    prints the summary of each and one JSON line with the last."""
    import ctypes
    lib = pa.load()
    if not hasattr(lib, "pa_timeline_copy"):
        sys.exit("--op timeline needs a library built with -DPA_TIMELINE "
                 "(python -m paged_kv_cache_222_amd.build --out=PATH "
                 "-DPA_TIMELINE), named by PA_LIBRARY")
    lib.pa_timeline_copy.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.pa_timeline_copy.restype = ctypes.c_int
    lib.pa_timeline_clear.restype = ctypes.c_int
    n_groups, n_slots, n_items = 4096, 64, 18
    kw = {"block_size": args.block_size} if args.block_size else {}
    w = wl.make_workload(args.config, seed=args.seed, **kw)
    c = w.cfg
    P = args.partition_size or c.partition_size
    form = args.variant if args.variant in ("fused", "split", "partitioned",
                                            "prefix") else (
        "prefix" if c.prefix_len else "fused")
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[c.dtype]

    def up(x, dt=None):
        if dt is not None:
            return torch.from_numpy(x.view(np.int16)).view(dt).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    copies = [dict(k=up(w.k_pool, tdt), v=up(w.v_pool, tdt))
              for _ in range(n_copies(args, w))]
    q, kn, vn = up(w.q, tdt), up(w.key_new, tdt), up(w.value_new, tdt)
    tbl, cl = up(w.block_table), up(w.context_lens)
    if form == "split":
        pm = args.slots or split_slots(w, torch)
    else:
        pm = max(1, -(-int(w.context_lens.max()) // P))
    ws = pa.partition_workspace(c.batch, c.n_q_heads, c.d_head, pm)

    def launch(x):
        if form == "fused":
            pa.pa_decode_step(*ws, kn, vn, q, x["k"], x["v"], tbl, cl,
                              partition_size=P, scale=w.scale)
        elif form == "split":
            pa.pa_decode_split(*ws, q, x["k"], x["v"], tbl, cl, scale=w.scale,
                               key_new=kn, value_new=vn)
        elif form == "prefix":
            pa.pa_decode_shared_prefix(*ws, q, x["k"], x["v"], tbl, cl,
                                       partition_size=P,
                                       prefix_len=c.prefix_len, scale=w.scale,
                                       key_new=kn, value_new=vn)
        else:
            pa.pa_decode_partitioned(*ws, q, x["k"], x["v"], tbl, cl,
                                     partition_size=P, scale=w.scale)

    for i in range(args.warmup):
        launch(copies[i % len(copies)])
    torch.cuda.synchronize()
    runs = []
    for i in range(args.steps):
        if lib.pa_timeline_clear() != 0:
            sys.exit("pa_timeline_clear failed")
        torch.cuda.synchronize()
        launch(copies[i % len(copies)])
        torch.cuda.synchronize()
        buf = np.zeros(n_groups * n_slots, dtype=np.uint64)
        if lib.pa_timeline_copy(buf.ctypes.data, buf.nbytes) != 0:
            sys.exit("pa_timeline_copy failed")
        runs.append(buf.reshape(n_groups, n_slots).astype(np.int64))

    def summary(t):
        t = t[t[:, 0] > 0]
        t0 = t[:, 0].min()
        us = lambda x: (x - t0) / 100.0           # 100 MHz ticks
        st, pl, en = us(t[:, 0]), us(t[:, 1]), us(t[:, 2])
        nit = t[:, 3]
        xcc = (t[:, 60] >> 32) & 0xF
        hw = t[:, 60] & 0xFFFFFFFF
        # HW_ID: CU id bits 8-11, shader array bit 12, shader engine 13-15
        cu_key = xcc * 256 + ((hw >> 8) & 0xFF)
        firsts, seconds = [], []
        for key in np.unique(cu_key):
            idx = np.where(cu_key == key)[0]
            if len(idx) == 2:
                i0, i1 = idx[np.argsort(st[idx])]
                firsts.append(en[i0])
                seconds.append(en[i1])
        durs, tiles, gaps = [], [], []
        wg_tiles = np.zeros(len(t))
        for g in range(len(t)):
            prev = None
            for k in range(min(n_items, int(nit[g]))):
                s0, s1, info = t[g, 4 + 3 * k], t[g, 5 + 3 * k], t[g, 6 + 3 * k]
                durs.append((s1 - s0) / 100.0)
                tiles.append(info & 0xFFFFF)
                wg_tiles[g] += info & 0xFFFFF
                if prev is not None:
                    gaps.append((s0 - prev) / 100.0)
                prev = s1
        # each CU's tiles (all its work groups' items, when every item was
        # recorded) and its end (its last work group's)
        cu_tiles, cu_end = [], []
        if (nit <= n_items).all():
            for key in np.unique(cu_key):
                idx = np.where(cu_key == key)[0]
                cu_tiles.append(wg_tiles[idx].sum())
                cu_end.append(en[idx].max())
        fit = [None, None]
        if len(durs) > 2 and np.ptp(tiles) > 0:
            A = np.vstack([np.ones(len(tiles)), np.array(tiles, float)]).T
            fit = [round(float(x), 3) for x in
                   np.linalg.lstsq(A, np.array(durs), rcond=None)[0]]
        phases = None
        if (t[:, 58] > 0).all() and (t[:, 61] > 0).all():
            # plan phases after a work group's start (p50): context lengths
            # in, after the scans, after the rank, the plan's end
            phases = [round(float(np.median(us(t[:, k]) - st)), 2)
                      for k in (58, 59, 61)] + \
                     [round(float(np.median(pl - st)), 2)]
        return {
            "work_groups": int(len(t)),
            "span_us": round(float(en.max()), 2),
            "start_us_p50_max": [round(float(np.median(st)), 2),
                                 round(float(st.max()), 2)],
            "plan_end_after_start_us_p50": round(float(np.median(pl - st)), 2),
            "plan_phases_us_p50_lengths_scan_rank_end": phases,
            "end_us_p0_p10_p50_p90_max": [round(float(x), 1) for x in
                                          np.percentile(en, [0, 10, 50, 90, 100])],
            "items_per_group_mean_max": [round(float(nit.mean()), 2),
                                         int(nit.max())],
            "xcc_median_end_us": [round(float(np.median(en[xcc == x])), 1)
                                  for x in range(8) if (xcc == x).any()],
            "cu_pairs": len(firsts),
            "cu_pair_end_us_first_second_p50":
                [round(float(np.median(firsts)), 1),
                 round(float(np.median(seconds)), 1)] if firsts else None,
            "cu_tiles_min_max": [int(min(cu_tiles)), int(max(cu_tiles))]
                                if cu_tiles else None,
            "cu_end_tiles_corr": round(float(np.corrcoef(cu_tiles, cu_end)[0, 1]), 2)
                                 if cu_tiles and np.ptp(cu_tiles) > 0 else None,
            "item_us_fixed_per_tile": fit,
            "gap_between_items_us_p50":
                round(float(np.median(gaps)), 2) if gaps else None,
        }

    for i, t in enumerate(runs):
        log(f"launch {i}: {json.dumps(summary(t))}")
    print(json.dumps({"op": "timeline", "config": c.name, "form": form,
                      "partition_size": P if form != "split" else None,
                      "slots": pm, "launches": len(runs),
                      "spans_us": [summary(t)["span_us"] for t in runs],
                      "last": summary(runs[-1])}), flush=True)


def bench_prefix_cache(args):
    """Host-side prefix caching on the shared-prefix batch: each of the 256
    requests (a 2048-token shared prompt + a private suffix U[1, 6144], token
    ids synthetic) is hashed block by block and mapped onto the pool; the
    first request creates the shared blocks, the rest hit them.  Also the
    Serving 23.4 widget under both policies."""
    import paged_kv_cache_222_amd as pa
    from paged_kv_cache_222_amd import pool_sim
    from paged_kv_cache_222_amd import workloads as wl
    c = wl.CONFIGS["shared-prefix"]
    bs = c.block_size
    ctx = wl.draw_lengths(c, args.seed)
    rng = np.random.default_rng(args.seed + 11)
    prompt = rng.integers(0, 128000, c.prefix_len).astype(np.int32)
    reqs = [np.concatenate([prompt, rng.integers(0, 128000, int(n) - c.prefix_len)
                            .astype(np.int32)]) for n in ctx]
    n_tok = int(sum(len(r) for r in reqs))
    blocks_needed = sum(-(-len(r) // bs) for r in reqs)

    def one_pass():
        pool = pa.pa_pool_create(blocks_needed)
        hits = 0
        tables = []
        for r in reqs:
            h = pa.pa_block_hashes(r, bs)
            ids, hit = pa.pa_pool_map_prefix(pool, h)
            tail = pa.pa_pool_alloc(pool, 1) if len(r) % bs else ids[:0]
            tables.append(np.concatenate([ids, tail]))
            hits += hit
        return hits, tables

    for _ in range(max(1, args.warmup // 5)):
        one_pass()
    reps = max(1, args.steps // 20)
    t0 = time.perf_counter()
    for _ in range(reps):
        hits, tables = one_pass()
    dt = (time.perf_counter() - t0) / reps
    shared = c.prefix_len // bs
    assert all((t[:shared] == tables[0][:shared]).all() for t in tables)
    W = wl.WIDGET
    a, pr, fi = wl.widget_requests(args.seed)
    sims = {pol: pool_sim.simulate(a, pr, fi, W["n_blocks"], W["block_size"],
                                   pol, W["max_len"])
            for pol in ("reserve", "paged")}
    rec = {
        "metric": "prefix-cache mapping requests/s (host, native: block "
                  "hashes + pool mapping)",
        "value": round(len(reqs) / dt, 1), "unit": "requests/s",
        "n_gpus": 0, "steps": reps, "warmup": max(1, args.warmup // 5),
        "ms_per_step": round(dt * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int32/uint64",
        "data": "synthetic",
        "config": {"workload": "shared-prefix batch: 256 requests, 2048-token "
                               "shared prompt + suffix U[1,6144], 16-token "
                               "blocks, one pass = hash + map every request",
                   "requests": len(reqs), "tokens": n_tok, "seed": args.seed},
        "tokens_hashed_per_s": round(n_tok / dt, 1),
        "prefix_hits": hits, "blocks_mapped": int(sum(len(t) for t in tables)),
        "widget": {pol: {"max_running": max(r["running"]),
                         "starts": r["start"],
                         "utilisation": round(r["utilisation"], 4)}
                   for pol, r in sims.items()},
        "roofline": None,
    }
    if not args.no_cpu_baseline:
        import oracle.block_pool as ob
        t0 = time.perf_counter()
        done = 0
        pool = ob.OraclePool(blocks_needed)
        while done < len(reqs) and time.perf_counter() - t0 < min(args.cpu_seconds, 10.0):
            pool.map_prefix(ob.block_hashes(reqs[done].tolist(), bs))
            done += 1
        dt2 = time.perf_counter() - t0
        rec["cpu_baseline"] = {
            "value": round(done / dt2, 3), "unit": "requests/s", "cores": 1,
            "kind": "oracle",
            "sample": f"first {done} of {len(reqs)} requests through the "
                      f"pure-Python oracle, {dt2:.1f} s"}
    print(json.dumps(rec), flush=True)


def cpu_baseline(w, budget_s):
    """The fp64 oracle on the host cores, over the first sequences of the
    batch (all query heads) until the time budget is spent."""
    import oracle
    c = w.cfg
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()]
                      or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    k_ref, v_ref = oracle.oracle_cache_write(w.k_pool, w.v_pool, w.key_new,
                                             w.value_new, w.slot_mapping,
                                             c.block_size)
    nbytes = {"f32": 4, "f16": 2, "bf16": 2}[c.dtype]

    def run(budget):
        t0 = time.perf_counter()
        done, kv = 0, 0
        for b in range(c.batch):
            oracle.oracle_decode(w.q, k_ref, v_ref, w.block_table,
                                 w.context_lens, w.scale, c.gqa_group,
                                 c.block_size, c.dtype,
                                 rows=[(b, h) for h in range(c.n_q_heads)])
            done += 1
            kv += int(w.context_lens[b]) * c.n_kv_heads * c.d_head * 2 * nbytes
            if time.perf_counter() - t0 > budget:
                break
        return done, kv, time.perf_counter() - t0

    done, kv, dt = run(budget_s)
    rec = {"value": round(kv / dt / 1e9, 4), "unit": "GB/s",
           "seq_steps_per_s": round(done / dt, 3), "cores": int(threads),
           "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
           "sample": f"first {done} of {c.batch} sequences, all "
                     f"{c.n_q_heads} query heads, fp64 numpy, {dt:.1f} s"}
    try:   # the same oracle with its BLAS on one thread
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            done1, kv1, dt1 = run(budget_s / 2)
        rec["one_thread"] = {
            "value": round(kv1 / dt1 / 1e9, 4), "unit": "GB/s",
            "seq_steps_per_s": round(done1 / dt1, 3), "cores": 1,
            "sample": f"first {done1} of {c.batch} sequences, {dt1:.1f} s"}
    except Exception:  # noqa: BLE001
        pass
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not "
              "supported (the decode path shards by sequence or KV head with "
              "no exchange, so N GPUs would run N independent copies)",
              file=sys.stderr)
        sys.exit(2)
    if args.op == "prefix-cache":
        bench_prefix_cache(args)
        return
    import torch

    import paged_kv_cache_222_amd as pa
    from paged_kv_cache_222_amd import workloads as wl

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    pa.load()
    if args.op == "copy-blocks":
        bench_copy_blocks(args, torch, pa, wl)
        return
    if args.op == "verify":
        bench_verify(args, torch, pa, wl)
        return
    if args.op == "timeline":
        bench_timeline(args, torch, pa, wl)
        return
    kw = {}
    if args.block_size:
        kw["block_size"] = args.block_size
    t = time.perf_counter()
    w = wl.make_workload(args.config, seed=args.seed, **kw)
    c = w.cfg
    P = args.partition_size or c.partition_size
    pmax = max(1, -(-int(w.context_lens.max()) // P))
    log(f"generated {c.name} in {time.perf_counter() - t:.1f}s: B={c.batch} "
        f"Hq={c.n_q_heads} Hkv={c.n_kv_heads} D={c.d_head} BS={c.block_size} "
        f"{c.dtype} sum(ctx)={int(w.context_lens.sum())} P={P} PMAX={pmax}")

    tdt = {"f32": torch.float32, "f16": torch.float16,
           "bf16": torch.bfloat16}[c.dtype]

    def up(x, dt=None):
        if dt == torch.bfloat16:
            return torch.from_numpy(x.view(np.int16)).view(tdt).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    copies = []
    for i in range(n_copies(args, w)):
        copies.append(dict(k=up(w.k_pool, tdt), v=up(w.v_pool, tdt),
                           q=up(w.q, tdt), kn=up(w.key_new, tdt),
                           vn=up(w.value_new, tdt)))
    tbl, cl, slots = up(w.block_table), up(w.context_lens), up(w.slot_mapping)
    out = torch.empty_like(copies[0]["q"])
    ws = pa.partition_workspace(c.batch, c.n_q_heads, c.d_head, pmax)
    n_slots = args.slots or split_slots(w, torch)
    ws_split = pa.partition_workspace(c.batch, c.n_q_heads, c.d_head, n_slots)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step(x, variant, ev=None):
        """One decode step; with ``ev`` (six events) it records the step's
        start, the end of the separate write, the ends of the attention and
        the reduce calls, and -- through pa_time_next_attention -- the
        attention kernel's own start and end."""
        if ev is not None:
            ev[0].record(stream)
        if variant in ("fused", "prefix", "split"):
            # the cache write happens inside the attention launch
            if ev is not None:
                ev[1].record(stream)
                pa.pa_time_next_attention(ev[4], ev[5])
            if variant == "fused":
                pa.pa_decode_step(*ws, x["kn"], x["vn"], x["q"], x["k"],
                                  x["v"], tbl, cl, partition_size=P,
                                  scale=w.scale)
            elif variant == "split":
                pa.pa_decode_split(*ws_split, x["q"], x["k"], x["v"], tbl, cl,
                                   scale=w.scale, key_new=x["kn"],
                                   value_new=x["vn"])
            else:
                # the shared prompt's partitions computed for several
                # sequences per work item
                pa.pa_decode_shared_prefix(
                    *ws, x["q"], x["k"], x["v"], tbl, cl, partition_size=P,
                    prefix_len=c.prefix_len, scale=w.scale,
                    key_new=x["kn"], value_new=x["vn"])
            if ev is not None:
                ev[2].record(stream)
            if variant == "split":
                pa.pa_reduce(out, *ws_split, cl, partition_size=0)
            else:
                pa.pa_reduce(out, *ws, cl, partition_size=P)
            if ev is not None:
                ev[3].record(stream)
            return
        pa.pa_cache_write(x["kn"], x["vn"], x["k"], x["v"], slots)
        if ev is not None:
            ev[1].record(stream)
            pa.pa_time_next_attention(ev[4], ev[5])
        if variant == "single":
            pa.pa_decode(out, x["q"], x["k"], x["v"], tbl, cl, scale=w.scale)
            if ev is not None:
                ev[2].record(stream)
        else:
            # "vector": the same launch on the vector-ALU kernel
            pa.pa_decode_partitioned(*ws, x["q"], x["k"], x["v"], tbl, cl,
                                     partition_size=P, scale=w.scale,
                                     vector=variant == "vector")
            if ev is not None:
                ev[2].record(stream)
            pa.pa_reduce(out, *ws, cl, partition_size=P)
        if ev is not None:
            ev[3].record(stream)

    def timed(variant):
        for i in range(args.warmup):
            step(copies[i % len(copies)], variant)
        torch.cuda.synchronize()
        # the timed region: exactly --steps steps, nothing else
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(copies[i % len(copies)], variant)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # the same steps again with events around each kernel
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)]
               for _ in range(args.steps)]
        for i in range(args.steps):
            step(copies[i % len(copies)], variant, evs[i])
        torch.cuda.synchronize()
        # microseconds: write, attention call, reduce call, whole step, and
        # the attention kernel itself (its dispatch's own timestamps)
        per = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]),
                         e[2].elapsed_time(e[3]), e[0].elapsed_time(e[3]),
                         e[4].elapsed_time(e[5])]
                        for e in evs]) * 1e3
        return wall, per

    variants = (["fused", "split", "partitioned", "single"]
                if args.variant in ("all", "best") else [args.variant])
    if c.prefix_len and args.variant in ("all", "best"):
        variants.insert(0, "prefix")
    if c.dtype == "f32" and "split" in variants and args.variant != "split":
        variants.remove("split")            # 16-bit types only
    if args.variant == "prefix" and not c.prefix_len:
        sys.exit("--variant prefix needs a batch with a shared prefix")
    results = {}
    for v in variants:
        log(f"timing {v}: warmup {args.warmup}, steps {args.steps}")
        wall, per = timed(v)
        results[v] = (wall, per)
        log(f"{v}: {wall / args.steps * 1e3:.4f} ms/step wall; us: write "
            f"{per[:, 0].mean():.1f} attention call {per[:, 1].mean():.1f} "
            f"(kernel {per[:, 4].mean():.1f}) reduce {per[:, 2].mean():.1f}")
    headline = "prefix" if c.prefix_len else HEADLINE_FORM.get(c.name, "fused")
    best = (min(results, key=lambda v: results[v][0]) if args.variant == "best"
            else headline if args.variant == "all" else args.variant)
    wall, per = results[best]
    ms = wall / args.steps * 1e3
    kv = w.kv_bytes_logical()
    uniq = w.kv_bytes_unique() if c.prefix_len else kv
    gbs = kv / (ms * 1e-3) / 1e9
    attn_us = float(per[:, 4].mean())      # the kernel's own timestamps
    alg = algorithmic_bytes(w)
    if c.prefix_len:
        alg = alg - kv + uniq
    if best in ("fused", "prefix", "split"):   # the new rows are read and written by the same launch
        alg += 2 * 2 * c.batch * c.n_kv_heads * c.d_head * \
            {"f32": 4, "f16": 2, "bf16": 2}[c.dtype]
    achieved = alg / (attn_us * 1e-6) / 1e9
    kernel = {"fused": "attention_mfma_kernel (pa_decode_step)",
              "split": "attention_mfma_kernel (pa_decode_split)",
              "prefix": "attention_mfma_kernel (pa_decode_shared_prefix)",
              "partitioned": "attention_mfma_kernel (pa_decode_partitioned)",
              "single": "attention_mfma_kernel (pa_decode)",
              "vector": "attention_kernel, vector ALU "
                        "(pa_decode_partitioned_vector)"}[best]
    rec = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic",
        "config": {"workload": f"{c.name} decode step (cache write + "
                               f"attention), one layer: {c.description}",
                   "batch": c.batch, "n_q_heads": c.n_q_heads,
                   "n_kv_heads": c.n_kv_heads, "d_head": c.d_head,
                   "block_size": c.block_size, "partition_size": P,
                   "sum_context": int(w.context_lens.sum()),
                   "seed": args.seed, "variant": best,
                   "split_slots": n_slots if best == "split" else None},
        "seq_steps_per_s": round(c.batch / (ms * 1e-3), 1),
        "pct_of_hbm_peak": round(100 * (uniq / (ms * 1e-3) / 1e9)
                                 / HBM_PEAK_GBS, 2),
        "kv_bytes_per_step": kv,
        "kv_bytes_unique_per_step": uniq,
        "kernel_us": {"cache_write": (None if best in ("fused", "prefix", "split")
                                      else round(float(per[:, 0].mean()), 2)),
                      "attention": round(attn_us, 2),
                      "attention_call_events": round(float(per[:, 1].mean()), 2),
                      "reduce": round(float(per[:, 2].mean()), 2),
                      "step_events": round(float(per[:, 3].mean()), 2),
                      "step_events_p10_p50_p90": [
                          round(float(x), 2) for x in
                          np.percentile(per[:, 3], [10, 50, 90])]},
        "variants_ms_per_step": {v: round(results[v][0] / args.steps * 1e3, 5)
                                 for v in results},
        "roofline": {"kernel": kernel, "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(c.name, best, P, c.block_size),
                     "algorithmic_bytes_per_launch": alg,
                     "avg_launch_us": round(attn_us, 3)},
    }
    # the pages' own figures, with their hardware (context, not a target:
    # none of them is a kernel rate on comparable hardware)
    rec["context"] = {
        "kv_cache_step": "4.7 s -> 65 ms per generated token at 4,096 tokens "
                         "with the cache kept (whole Qwen2.5-1.5B-Instruct "
                         "model, a laptop)",
        "pool_utilisation": "90-98% of reserved KV memory holds tokens with "
                            "16-token blocks and a block table, against "
                            "3-63% for worst-case contiguous reservation "
                            "(ShareGPT/Alpaca requests, memory accounting)"}
    if not args.no_read_ceiling:
        log("measuring the read ceiling (4 GiB, stream and 4 KiB-tile gather)")
        del copies
        rc = measure_read_ceiling(torch, pa, batch_tiles=uniq // 4096)
        rc["attention_frac_of_tile_gather"] = round(
            achieved / rc["tile_gather_GBs"], 4)
        if "batch_size_tile_gather_GBs" in rc:
            rc["attention_frac_of_batch_size_gather"] = round(
                achieved / rc["batch_size_tile_gather_GBs"], 4)
        rec["read_ceiling"] = rc
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle on a sample")
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
