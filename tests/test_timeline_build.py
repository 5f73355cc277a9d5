"""The measurement build of the matrix-core kernel (-DPA_TIMELINE, read by
bench.py --op timeline) still compiles for gfx950, and the product build
carries none of it (no timeline symbols exported).  CPU only."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_222_amd", "csrc")


def test_timeline_build_compiles(tmp_path):
    from paged_kv_cache_222_amd import build as B
    cc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cc):
        pytest.skip("hipcc not available")
    obj = tmp_path / "tl.o"
    cmd = [cc, *B.HIP_FLAGS, "-DPA_TIMELINE", f"-I{B.INCLUDE}", f"-I{CSRC}",
           "-c", os.path.join(CSRC, "pa_attention_mfma.hip"), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    syms = subprocess.run(["nm", "--defined-only", str(obj)],
                          capture_output=True, text=True).stdout
    assert "pa_timeline_copy" in syms and "pa_timeline_clear" in syms


def test_product_build_has_no_timeline():
    from paged_kv_cache_222_amd import _binding
    path = _binding.library_path()
    if not os.path.exists(path):
        pytest.skip("library not built")
    syms = subprocess.run(["nm", "-D", "--defined-only", path],
                          capture_output=True, text=True).stdout
    assert "pa_timeline" not in syms
