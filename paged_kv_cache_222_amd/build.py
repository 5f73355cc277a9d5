"""Build libpa.so: the HIP kernels and the C ABI, for gfx950.

Run ``python -m paged_kv_cache_222_amd.build`` (or ``build()``).  Each
``csrc/*.hip`` file is compiled to an object in ``_build/`` in parallel with
hipcc, then linked into ``paged_kv_cache_222_amd/libpa.so``.  Always
recompiles: the build is the check that the sources compile.
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"

# -packed-fp32-ops: never emit packed fp32 VALU ops (v_pk_{add,mul,fma}_f32).
# -amdgpu-mfma-vgpr-form: MFMA accumulators in VGPRs, so the softmax rescale
# of the accumulators needs no copies between register files.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"),
                 "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required)")


def _compile(src: str, cc: str, extra, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [cc, *HIP_FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}", "-c", src,
           "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n"
                           f"{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Compile every HIP source and link libpa.so (or ``out``); returns its
    path."""
    cc = hipcc()
    build_dir = BUILD_DIR if out == LIB else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, cc, list(extra_flags), build_dir),
                           srcs))
    for src in sorted(glob.glob(os.path.join(CSRC, "*.cpp"))):   # host-only code
        obj = os.path.join(build_dir, os.path.basename(src)[:-4] + ".o")
        cmd = ["g++", *CXX_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"g++ failed for {src}:\n{' '.join(cmd)}\n"
                               f"{res.stdout}\n{res.stderr}")
        objs.append(obj)
        srcs.append(src)
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n"
                           f"{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(srcs)} sources")
    return out


if __name__ == "__main__":
    args = sys.argv[1:]
    out = LIB
    if args and args[0].startswith("--out="):
        out = os.path.abspath(args.pop(0)[len("--out="):])
    build(verbose=True, extra_flags=args, out=out)
