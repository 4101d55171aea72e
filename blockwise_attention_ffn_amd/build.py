"""Build the gfx950 shared library libbpt.so in-tree with hipcc.

Usage: python -m blockwise_attention_ffn_amd.build   (or call build()).
Every call recompiles; objects go to _build/ next to the package.
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
LIB = os.path.join(PKG, "libbpt.so")

SOURCES = ["bpt_api.cpp", "gemm_bf16.hip", "attn_bf16.hip", "attn_bwd.hip", "fp32_path.hip", "dropout.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # no packed fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-file flags. The attention kernel runs with the IEEE mode bit off: its
# min/max then need no NaN-quieting of MFMA results (it produces no NaN: masked
# scores are -inf and every maximum it takes is finite).
# The attention backward keeps its score blocks and gradient accumulators in
# VGPRs (the element-wise work reads the score blocks every step; in the AGPR
# form each read and each starting value would be a v_accvgpr move) and
# holds its constant MFMA B operands in AGPRs.
PER_FILE = {"attn_bf16.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"],
            "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    errs = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    return obj


def build(verbose: bool = True, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
