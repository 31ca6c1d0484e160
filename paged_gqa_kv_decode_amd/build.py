"""Build libvkpaged.so in-tree with hipcc for gfx950.

    python -m paged_gqa_kv_decode_amd.build

Every HIP translation unit is compiled with packed-fp32 instruction
generation disabled (`-Xclang -target-feature -Xclang -packed-fp32-ops`);
hipcc's host pass warns that it does not know that feature, which is
harmless.  Object files go to `_build/` (git-ignored); the shared library is
written next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libvkpaged.so")
BENCH_LIB = os.path.join(PKG, "libvkbench.so")   # measurement-only kernels
ARCH = "gfx950"

SOURCES = ["vk_host.cpp", "decode_dot.hip", "decode_mfma.hip", "decode_mfma_mhq.hip",
           "decode_mfma_bf16.hip", "decode_mfma_f32.hip", "decode_varlen.hip",
           "decode_varlen_tile.hip", "reduce.hip",
           "kv_append.hip", "noalloc.hip"]
BENCH_SOURCES = ["bench_kernels.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]


# Per-source flags.  The LDS-tiled multi-token kernel keeps its matrix-core
# accumulators in VGPRs: with the default AGPR form the compiler copied all
# of them out of AGPRs on every key tile for the (rarely taken) softmax
# rescale.
EXTRA = {"decode_varlen_tile.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), *lang, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed for {src}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(_compile, SOURCES + BENCH_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], BENCH_LIB)
    if verbose:
        print("built", LIB, "and", BENCH_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
