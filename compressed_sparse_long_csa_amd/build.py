"""Build libcsa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m compressed_sparse_long_csa_amd.build
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libcsa.so")
SOURCES = ["csa_abi.hip", "compress.hip", "indexer.hip", "score_topk.hip", "topk.hip", "attn.hip", "cp_gather.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # LDS buffers are written and read through different types (packed
    # words, vectors, byte pointers): no type-based alias assumptions
    "-fno-strict-aliasing",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-command-line-argument",
]
# per-file additions: the indexer and the attention keep MFMA results in
# VGPRs (the indexer's head sum reads every result element; the attention's
# accumulators are rescaled by VALU, and AGPR-held results would be copied
# through VGPRs at every loop iteration)
EXTRA = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "score_topk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         # the ILP scheduler batches each step's operand reads ahead of its
         # MFMAs (one wave per SIMD has no other wave to hide LDS latency)
         "attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def _compile(src):
    obj = os.path.join(LIBDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose=False):
    os.makedirs(LIBDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
