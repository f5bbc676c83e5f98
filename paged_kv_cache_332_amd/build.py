"""Build libpa.so (HIP for gfx950) in place: ``python paged_kv_cache_332_amd/build.py``.

Each translation unit is compiled by hipcc in parallel into ``_build/`` and
linked into ``paged_kv_cache_332_amd/libpa.so``.  Packed-FP32 instruction
selection is switched off for device code (the compiler still uses scalar
fp32 FMAs).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if p and os.path.exists(p):
            return p
    raise RuntimeError("hipcc not found")


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-file additions.  The decode kernels keep their matrix-core
# accumulators in VGPRs: with the default heuristic they live in AGPRs and
# the compiler copies all 32 of them between the two register files in every
# tile's softmax and at the loop head (about 100 v_accvgpr moves per 16-token
# tile, more than the tile's own vector work), read off the gfx950 assembly.
FILE_FLAGS = {f: ["-mllvm", "-amdgpu-mfma-vgpr-form"] for f in ("decode_stream.hip", "decode_mfma.hip")}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    # the host microbenchmark of the block manager's calls, linked to the library
    tool = os.path.join(PKG, "bm_bench")
    cmd = [shutil.which("g++") or "g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           os.path.join(PKG, "bm_bench.cpp"), "-o", tool + ".tmp", "-L", PKG, "-lpa", "-Wl,-rpath,$ORIGIN",
           "-Wl,--allow-shlib-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"host tool build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tool + ".tmp", tool)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
