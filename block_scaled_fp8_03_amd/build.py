"""Build libfp8bs.so (gfx950) in-tree with hipcc.

Usage: python -m block_scaled_fp8_03_amd.build   (or build() from Python)

Every HIP source is compiled for gfx950 only, with packed-FP32 instructions
disabled and floating-point contraction off (the kernels write every FMA they
want explicitly), then linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfp8bs.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["quant.hip", "gemm.hip", "gemm_e8.hip", "moe_dispatch.hip", "mla.hip", "abi.cpp"]

COMMON_FLAGS = [
    "-std=c++17", "-O3", "-fPIC", "-Wall", "-Wno-unused-function",
    "-ffp-contract=off",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# MFMA results in VGPRs: the per-K-block scale fold reads them with VALU FMAs,
# which cannot take AGPR operands.  gemm_e8.hip has no fold and keeps its 256
# accumulators per lane in AGPRs, so it is built without this.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
AGPR_SOURCES = {"gemm_e8.hip"}


def _compile(src: str, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    form = [] if src in AGPR_SOURCES else VGPR_FORM
    cmd = [HIPCC, *COMMON_FLAGS, *HIP_FLAGS, *form, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *COMMON_FLAGS, "--offload-arch=gfx950", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
