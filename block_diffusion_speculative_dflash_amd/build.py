"""Build the gfx950 HIP libraries in-tree with hipcc.

libdflash.so          the C-ABI library (include/dflash.h): api + kernels
libdflash_harness.so  the benchmark's target stand-in (planted targets)

Run ``python -m block_diffusion_speculative_dflash_amd.build`` (or
``__graft_entry__.build()``); it always recompiles.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdflash.so")
HARNESS_LIB = os.path.join(PKG, "libdflash_harness.so")

LIB_SOURCES = ["api.hip", "gemm.hip", "gemm_tiled.hip", "attention.hip", "misc.hip", "pack.hip", "sampling.hip",
               "persist.hip"]
HARNESS_SOURCES = ["harness_plant.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU instructions are disabled for all device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


# Per-source flags.  attention.hip: MFMA accumulators in VGPRs, so the online-softmax
# rescale of the output accumulators needs no moves between AGPRs and VGPRs.
SOURCE_FLAGS = {"attention.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
                "persist.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for {out}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> None:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = LIB_SOURCES + HARNESS_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in LIB_SOURCES], LIB)
    _link([objs[s] for s in HARNESS_SOURCES], HARNESS_LIB)
    if verbose:
        print(f"built {LIB} and {HARNESS_LIB}", file=sys.stderr)


if __name__ == "__main__":
    build()
