"""The C ABI: the library loads, exports what include/pa.h declares, and
rejects bad host-side arguments before touching the GPU (no compute calls
here, so these run without a GPU)."""

import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED = 0, -1, -2, -3
PA_ERR_WORKSPACE, PA_ERR_PARTITION, PA_ERR_HIP, PA_ERR_ALIGN = -4, -5, -6, -7
PA_ERR_NOSPACE, PA_ERR_SCRATCH = -8, -9

P = 0x100000        # a fake, 16-byte aligned device address (never touched)
MIS = P + 8         # misaligned


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pa_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(
        ["pa_block_hashes", "pa_cache_write", "pa_copy_blocks", "pa_decode",
         "pa_decode_multi", "pa_decode_partitioned",
         "pa_decode_partitioned_vector", "pa_decode_shared_prefix", "pa_decode_split", "pa_decode_step",
         "pa_decode_step_noalloc", "pa_pool_alloc",
         "pa_pool_available", "pa_pool_create", "pa_pool_destroy",
         "pa_pool_fork", "pa_pool_map_prefix", "pa_pool_refcount",
         "pa_pool_release", "pa_pool_simulate", "pa_read_ceiling",
         "pa_reduce", "pa_strerror", "pa_time_next_attention"])


def test_library_exports_every_declared_symbol(lib):
    from paged_kv_cache_222_amd import _binding
    out = subprocess.run(["nm", "-D", "--defined-only",
                          _binding.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_strerror_covers_every_status(lib):
    seen = set()
    for st in (PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED,
               PA_ERR_WORKSPACE, PA_ERR_PARTITION, PA_ERR_HIP, PA_ERR_ALIGN,
               PA_ERR_NOSPACE, PA_ERR_SCRATCH):
        text = lib.pa_strerror(st).decode()
        assert text and text != "unknown status"
        seen.add(text)
    assert len(seen) == 10
    assert lib.pa_strerror(12345).decode() == "unknown status"


def _cw(lib, **kw):
    a = dict(key=P, value=P, k_pool=P, v_pool=P, slots=P, n=4, hkv=2, d=128,
             bs=16, nb=8, dt=2)
    a.update(kw)
    return lib.pa_cache_write(a["key"], a["value"], a["k_pool"], a["v_pool"],
                              a["slots"], a["n"], a["hkv"], a["d"], a["bs"],
                              a["nb"], a["dt"], None)


def test_cache_write_argument_checks(lib):
    assert _cw(lib, n=0) == PA_OK                     # no-op, nothing launched
    assert _cw(lib, n=-1) == PA_ERR_SHAPE
    for k in ("key", "value", "k_pool", "v_pool", "slots"):
        assert _cw(lib, **{k: None}) == PA_ERR_NULL, k
    assert _cw(lib, d=96) == PA_ERR_UNSUPPORTED
    assert _cw(lib, bs=12) == PA_ERR_UNSUPPORTED
    assert _cw(lib, bs=128) == PA_ERR_UNSUPPORTED
    assert _cw(lib, dt=3) == PA_ERR_UNSUPPORTED
    assert _cw(lib, hkv=0) == PA_ERR_SHAPE
    assert _cw(lib, nb=0) == PA_ERR_SHAPE
    assert _cw(lib, key=MIS) == PA_ERR_ALIGN
    assert _cw(lib, k_pool=MIS) == PA_ERR_ALIGN


def _cb(lib, **kw):
    a = dict(k_pool=P, v_pool=P, pairs=P, n=4, hkv=2, d=128, bs=16, nb=8,
             dt=2)
    a.update(kw)
    return lib.pa_copy_blocks(a["k_pool"], a["v_pool"], a["pairs"], a["n"],
                              a["hkv"], a["d"], a["bs"], a["nb"], a["dt"],
                              None)


def test_copy_blocks_argument_checks(lib):
    assert _cb(lib, n=0) == PA_OK                     # no-op, nothing launched
    assert _cb(lib, n=-1) == PA_ERR_SHAPE
    for k in ("k_pool", "v_pool", "pairs"):
        assert _cb(lib, **{k: None}) == PA_ERR_NULL, k
    assert _cb(lib, d=48) == PA_ERR_UNSUPPORTED
    assert _cb(lib, bs=24) == PA_ERR_UNSUPPORTED
    assert _cb(lib, dt=5) == PA_ERR_UNSUPPORTED
    assert _cb(lib, hkv=0) == PA_ERR_SHAPE
    assert _cb(lib, nb=0) == PA_ERR_SHAPE
    assert _cb(lib, k_pool=MIS) == PA_ERR_ALIGN
    assert _cb(lib, pairs=P + 2) == PA_ERR_ALIGN
    assert _cb(lib, n=2**30, hkv=64, bs=64, dt=0) == PA_ERR_SHAPE  # launch grid


def _dec(lib, **kw):
    a = dict(out=P, q=P, k=P, v=P, tbl=P, mb=16, ctx=P, B=4, hkv=2, G=4,
             d=128, bs=16, nb=32, scale=0.1, dt=2)
    a.update(kw)
    return lib.pa_decode(a["out"], a["q"], a["k"], a["v"], a["tbl"], a["mb"],
                         a["ctx"], a["B"], a["hkv"], a["G"], a["d"], a["bs"],
                         a["nb"], a["scale"], a["dt"], None)


def test_decode_argument_checks(lib):
    assert _dec(lib, B=0) == PA_OK
    assert _dec(lib, B=-2) == PA_ERR_SHAPE
    for k in ("out", "q", "k", "v", "tbl", "ctx"):
        assert _dec(lib, **{k: None}) == PA_ERR_NULL, k
    assert _dec(lib, d=32) == PA_ERR_UNSUPPORTED
    assert _dec(lib, bs=4) == PA_ERR_UNSUPPORTED
    assert _dec(lib, dt=-1) == PA_ERR_UNSUPPORTED
    assert _dec(lib, G=0) == PA_ERR_SHAPE
    assert _dec(lib, hkv=0) == PA_ERR_SHAPE
    assert _dec(lib, mb=0) == PA_ERR_SHAPE
    assert _dec(lib, nb=0) == PA_ERR_SHAPE
    assert _dec(lib, mb=2**30) == PA_ERR_SHAPE        # max_blocks*bs overflows
    assert _dec(lib, q=MIS) == PA_ERR_ALIGN
    assert _dec(lib, out=MIS) == PA_ERR_ALIGN
    assert _dec(lib, tbl=P + 2) == PA_ERR_ALIGN


def _part(lib, fn="pa_decode_partitioned", **kw):
    a = dict(ml=P, es=P, to=P, psz=512, pmax=4, q=P, k=P, v=P, tbl=P, mb=64,
             ctx=P, B=4, hkv=2, G=4, d=128, bs=16, nb=32, scale=0.1, dt=2)
    a.update(kw)
    return getattr(lib, fn)(
        a["ml"], a["es"], a["to"], a["psz"], a["pmax"], a["q"], a["k"],
        a["v"], a["tbl"], a["mb"], a["ctx"], a["B"], a["hkv"], a["G"], a["d"],
        a["bs"], a["nb"], a["scale"], a["dt"], None)


@pytest.mark.parametrize("fn", ["pa_decode_partitioned",
                                "pa_decode_partitioned_vector"])
def test_partitioned_argument_checks(lib, fn):
    def call(**kw):
        return _part(lib, fn, **kw)
    assert call(B=0) == PA_OK
    for k in ("ml", "es", "to", "q", "tbl"):
        assert call(**{k: None}) == PA_ERR_NULL, k
    assert call(psz=0) == PA_ERR_PARTITION
    assert call(psz=24) == PA_ERR_PARTITION     # not a multiple of 16
    assert call(psz=-16) == PA_ERR_PARTITION
    assert call(pmax=0) == PA_ERR_WORKSPACE
    assert call(d=256) == PA_ERR_UNSUPPORTED
    assert call(to=MIS) == PA_ERR_ALIGN
    assert call(pmax=2**20, B=2**12) == PA_ERR_SHAPE   # grid too large


def _multi(lib, **kw):
    a = dict(ml=P, es=P, to=P, psz=512, pmax=4, q=P, k=P, v=P, tbl=P, mb=64,
             ctx=P, B=4, nq=4, hkv=2, G=4, d=128, bs=16, nb=32, scale=0.1,
             dt=2)
    a.update(kw)
    return lib.pa_decode_multi(
        a["ml"], a["es"], a["to"], a["psz"], a["pmax"], a["q"], a["k"],
        a["v"], a["tbl"], a["mb"], a["ctx"], a["B"], a["nq"], a["hkv"],
        a["G"], a["d"], a["bs"], a["nb"], a["scale"], a["dt"], None)


def test_multi_argument_checks(lib):
    assert _multi(lib, B=0) == PA_OK
    assert _multi(lib, nq=0) == PA_ERR_SHAPE
    for k in ("ml", "es", "to", "q", "k", "v", "tbl", "ctx"):
        assert _multi(lib, **{k: None}) == PA_ERR_NULL, k
    assert _multi(lib, dt=0) == PA_ERR_UNSUPPORTED        # fp32, k > 1
    assert _multi(lib, d=96) == PA_ERR_UNSUPPORTED
    assert _multi(lib, psz=24) == PA_ERR_PARTITION
    assert _multi(lib, pmax=0) == PA_ERR_WORKSPACE
    assert _multi(lib, to=MIS) == PA_ERR_ALIGN
    assert _multi(lib, nq=2**20, B=2**12) == PA_ERR_SHAPE  # rows overflow


def _step(lib, **kw):
    a = dict(ml=P, es=P, to=P, psz=512, pmax=4, kn=P, vn=P, q=P, k=P, v=P,
             tbl=P, mb=64, ctx=P, B=4, hkv=2, G=4, d=128, bs=16, nb=32,
             scale=0.1, dt=2)
    a.update(kw)
    return lib.pa_decode_step(
        a["ml"], a["es"], a["to"], a["psz"], a["pmax"], a["kn"], a["vn"],
        a["q"], a["k"], a["v"], a["tbl"], a["mb"], a["ctx"], a["B"], a["hkv"],
        a["G"], a["d"], a["bs"], a["nb"], a["scale"], a["dt"], None)


def test_step_argument_checks(lib):
    assert _step(lib, B=0) == PA_OK
    for k in ("ml", "es", "to", "kn", "vn", "q", "k", "v", "tbl", "ctx"):
        assert _step(lib, **{k: None}) == PA_ERR_NULL, k
    assert _step(lib, kn=MIS) == PA_ERR_ALIGN
    assert _step(lib, psz=8) == PA_ERR_PARTITION
    assert _step(lib, d=32) == PA_ERR_UNSUPPORTED


def _noalloc(lib, **kw):
    a = dict(out=P, psz=512, kn=P, vn=P, q=P, k=P, v=P, tbl=P, mb=64, ctx=P,
             B=4, hkv=2, G=4, d=128, bs=16, nb=32, scale=0.1, dt=2)
    a.update(kw)
    return lib.pa_decode_step_noalloc(
        a["out"], a["psz"], a["kn"], a["vn"], a["q"], a["k"], a["v"],
        a["tbl"], a["mb"], a["ctx"], a["B"], a["hkv"], a["G"], a["d"],
        a["bs"], a["nb"], a["scale"], a["dt"], None)


def test_noalloc_argument_checks(lib):
    """Every refusal comes before any HIP call (so these run without a
    GPU), the fixed buffer's limit included."""
    assert _noalloc(lib, B=0) == PA_OK
    for k in ("out", "kn", "vn", "q", "k", "v", "tbl", "ctx"):
        assert _noalloc(lib, **{k: None}) == PA_ERR_NULL, k
    assert _noalloc(lib, out=MIS) == PA_ERR_ALIGN
    assert _noalloc(lib, kn=MIS) == PA_ERR_ALIGN
    assert _noalloc(lib, psz=8) == PA_ERR_PARTITION
    assert _noalloc(lib, d=32) == PA_ERR_UNSUPPORTED
    assert _noalloc(lib, B=-1) == PA_ERR_SHAPE
    # 256 x 32 heads x ceil(8192 / 512) partitions x 130 floats = 68 MB
    assert _noalloc(lib, B=256, hkv=8, mb=512, psz=512) == PA_ERR_SCRATCH
    # exactly at the limit: 32 MiB = rows * pmax * 130 * 4 has no integer
    # solution, so check one row below and above it
    rows_fit = (32 << 20) // (130 * 4)               # with pmax = 1
    assert _noalloc(lib, B=rows_fit + 1, hkv=1, G=1, mb=32, psz=512) == \
        PA_ERR_SCRATCH


def _split(lib, **kw):
    a = dict(ml=P, es=P, to=P, pmax=8, kn=P, vn=P, q=P, k=P, v=P, tbl=P,
             mb=64, ctx=P, B=4, hkv=2, G=4, d=128, bs=16, nb=32, scale=0.1,
             dt=2)
    a.update(kw)
    return lib.pa_decode_split(
        a["ml"], a["es"], a["to"], a["pmax"], a["kn"], a["vn"], a["q"],
        a["k"], a["v"], a["tbl"], a["mb"], a["ctx"], a["B"], a["hkv"],
        a["G"], a["d"], a["bs"], a["nb"], a["scale"], a["dt"], None)


def test_split_argument_checks(lib):
    assert _split(lib, B=0) == PA_OK
    for k in ("ml", "es", "to", "q", "k", "v", "tbl", "ctx"):
        assert _split(lib, **{k: None}) == PA_ERR_NULL, k
    assert _split(lib, kn=None) == PA_ERR_NULL        # only as a pair
    assert _split(lib, kn=MIS) == PA_ERR_ALIGN
    assert _split(lib, to=MIS) == PA_ERR_ALIGN
    assert _split(lib, pmax=1) == PA_ERR_WORKSPACE    # at least two slots
    assert _split(lib, dt=0, d=64) == PA_ERR_UNSUPPORTED   # fp32
    assert _split(lib, d=32) == PA_ERR_UNSUPPORTED
    # tile counts must fit 32 bits
    assert _split(lib, B=1024, mb=1 << 20) == PA_ERR_SHAPE


def test_timing_hook_accepts_and_cancels(lib):
    assert lib.pa_time_next_attention(None, None) == PA_OK


def _prefix(lib, **kw):
    a = dict(ml=P, es=P, to=P, psz=512, pmax=4, kn=P, vn=P, q=P, k=P, v=P,
             tbl=P, mb=64, ctx=P, B=4, hkv=2, G=4, d=128, bs=16, nb=32,
             plen=512, scale=0.1, dt=2)
    a.update(kw)
    return lib.pa_decode_shared_prefix(
        a["ml"], a["es"], a["to"], a["psz"], a["pmax"], a["kn"], a["vn"],
        a["q"], a["k"], a["v"], a["tbl"], a["mb"], a["ctx"], a["B"], a["hkv"],
        a["G"], a["d"], a["bs"], a["nb"], a["plen"], a["scale"], a["dt"],
        None)


def test_shared_prefix_argument_checks(lib):
    assert _prefix(lib, B=0) == PA_OK
    for k in ("ml", "es", "to", "q", "k", "v", "tbl", "ctx"):
        assert _prefix(lib, **{k: None}) == PA_ERR_NULL, k
    # the new rows are optional, but only as a pair
    assert _prefix(lib, kn=None) == PA_ERR_NULL
    assert _prefix(lib, vn=None) == PA_ERR_NULL
    assert _prefix(lib, kn=MIS) == PA_ERR_ALIGN
    assert _prefix(lib, plen=-1) == PA_ERR_SHAPE
    assert _prefix(lib, psz=8) == PA_ERR_PARTITION
    assert _prefix(lib, pmax=0) == PA_ERR_WORKSPACE
    assert _prefix(lib, d=32) == PA_ERR_UNSUPPORTED


def _ceil(lib, **kw):
    a = dict(buf=P, nb=1 << 20, order=None, n=256, tb=4096, sink=P)
    a.update(kw)
    return lib.pa_read_ceiling(a["buf"], a["nb"], a["order"], a["n"], a["tb"],
                               a["sink"], None)


def test_read_ceiling_argument_checks(lib):
    assert _ceil(lib, n=0) == PA_OK
    assert _ceil(lib, n=-1) == PA_ERR_SHAPE
    assert _ceil(lib, buf=None) == PA_ERR_NULL
    assert _ceil(lib, sink=None) == PA_ERR_NULL
    assert _ceil(lib, tb=24) == PA_ERR_SHAPE
    assert _ceil(lib, tb=0) == PA_ERR_SHAPE
    assert _ceil(lib, n=257) == PA_ERR_SHAPE        # past the buffer, no order
    assert _ceil(lib, buf=MIS) == PA_ERR_ALIGN
    assert _ceil(lib, order=P + 2, n=300) == PA_ERR_ALIGN


def _red(lib, **kw):
    a = dict(out=P, ml=P, es=P, to=P, ctx=P, B=4, hq=8, d=128, psz=512,
             pmax=4, dt=2)
    a.update(kw)
    return lib.pa_reduce(a["out"], a["ml"], a["es"], a["to"], a["ctx"],
                         a["B"], a["hq"], a["d"], a["psz"], a["pmax"],
                         a["dt"], None)


def test_reduce_argument_checks(lib):
    assert _red(lib, B=0) == PA_OK
    for k in ("out", "ml", "es", "to", "ctx"):
        assert _red(lib, **{k: None}) == PA_ERR_NULL, k
    assert _red(lib, d=100) == PA_ERR_UNSUPPORTED
    assert _red(lib, dt=9) == PA_ERR_UNSUPPORTED
    assert _red(lib, hq=0) == PA_ERR_SHAPE
    assert _red(lib, psz=-1) == PA_ERR_PARTITION   # 0: a split workspace
    assert _red(lib, pmax=0) == PA_ERR_WORKSPACE
    assert _red(lib, out=MIS) == PA_ERR_ALIGN


def test_binding_fails_loudly_without_library(tmp_path):
    """With the library missing, the product path raises instead of
    computing anything another way."""
    env = dict(os.environ, PA_LIBRARY=str(tmp_path / "missing.so"))
    code = ("import paged_kv_cache_222_amd as p\n"
            "try:\n    p.load()\nexcept RuntimeError as e:\n"
            "    print('RAISED', e)\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env,
                         capture_output=True, text=True, check=True).stdout
    assert "RAISED" in out and "missing.so" in out


def test_binding_names_match_the_c_abi():
    import paged_kv_cache_222_amd as p
    for name in declared_functions():
        assert callable(getattr(p, name)), name


def test_product_code_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "paged_kv_cache_222_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, re.M), f
                assert "oracle/" not in text, f


def test_one_hip_runtime_in_the_process():
    """libpa must bind to the HIP runtime torch loads; two runtimes in one
    process make torch's streams invalid for libpa's launches."""
    code = ("import paged_kv_cache_222_amd as p\n"
            "p.load()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT,
                         capture_output=True, text=True, check=True).stdout
    assert out.strip() == "1"
