"""Build libmla.so (HIP, gfx950) in-tree with hipcc.

Each translation unit is compiled in parallel, then linked into
int2_quantized_absorbed_amd/libmla.so.  Run directly (python -m
int2_quantized_absorbed_amd.build_lib) or through __graft_entry__.build().
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla.so")

SOURCES = ["api.hip", "append.hip", "calib.hip", "decode.hip", "decode_mfma.hip", "gqa.hip", "index.hip",
           "splitk.hip"]
# Per-source flags.  The split-K kernel keeps its MFMA accumulators and
# operands in ordinary VGPRs (the VGPR form of MFMA): its two wave roles then
# fit in 256 registers each, two waves per SIMD.
SOURCE_FLAGS = {"splitk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
HOST_SOURCES = ["eigh.cpp"]

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + p.stdout)
    return p.stdout


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([cc, *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
