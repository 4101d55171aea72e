"""Build the gfx950 shared library libbpt.so in-tree with hipcc.

Usage: python -m blockwise_attention_ffn_amd.build   (or call build()).
Every call recompiles; objects go to _build/ next to the package.

Every source that includes csrc/lds_dma.h (kernels loading memory straight
into LDS, with hand-counted waits) is also compiled to assembly with the
compiler's resource-usage remarks, and the build fails unless each of its
kernels has no scratch memory, no spills, no out-of-line calls, no
vector-memory instruction but loads into LDS while such a load may be
outstanding, and the wait states before every descriptor or M0 read that the
compiler does not insert for inline asm (asm_check.py).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

try:
    from . import asm_check
except ImportError:  # run as a script
    import asm_check

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbpt.so")

SOURCES = ["bpt_api.cpp", "gemm_bf16.hip", "attn_bf16.hip", "attn_bf16_d32.hip", "attn_bf16_d64.hip",
           "attn_bf16_d128.hip", "attn_bwd.hip", "fp32_path.hip", "dropout.hip", "noalloc.hip"]

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
# The attention-forward variants with fewer waves per workgroup only bind
# the compiler to one wave per SIMD; they are kept in VGPR-form MFMAs (as the
# backward) and their issue-slot loops are unrolled in full (the default
# pragma threshold leaves the largest rolled, with its arrays in scratch).
_ATTN_FWD = ["-mno-amdgpu-ieee", "-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-mllvm", "-pragma-unroll-threshold=1000000"]
PER_FILE = {"attn_bf16_d32.hip": _ATTN_FWD, "attn_bf16_d64.hip": _ATTN_FWD,
            "attn_bf16_d128.hip": _ATTN_FWD,
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


def uses_lds_dma(src: str, _seen=None) -> bool:
    """True if src includes lds_dma.h, directly or through a local header."""
    import re
    seen = set() if _seen is None else _seen
    if src in seen:
        return False
    seen.add(src)
    with open(os.path.join(CSRC, src)) as fh:
        incs = re.findall(r'^#include "([^"]+)"', fh.read(), flags=re.M)
    return any(i == "lds_dma.h" or (os.path.exists(os.path.join(CSRC, i)) and uses_lds_dma(i, seen))
               for i in incs)


def check_source(src: str, extra=(), out_dir: str = BUILD):
    """Compile one source's device code to assembly with resource remarks and
    run the static checks. Returns (kernels checked, violations)."""
    asm = os.path.join(out_dir, os.path.splitext(src)[0] + ".gfx950.s")
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), *extra, "--cuda-device-only", "-S",
           "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src), "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    with open(asm) as fh:
        checked, errs = asm_check.check_asm_text(fh.read())
    errs = errs + asm_check.resource_violations(asm_check.parse_resource_remarks(r.stderr), checked)
    return checked, [f"{src}: {e}" for e in errs]


def build(verbose: bool = True, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    checked_srcs = [s for s in SOURCES if s.endswith(".hip") and uses_lds_dma(s)]
    jobs = min(len(SOURCES) + len(checked_srcs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, s, list(extra)) for s in SOURCES]
        chks = [ex.submit(check_source, s, list(extra)) for s in checked_srcs]
        objs = [f.result() for f in futs]
        results = [f.result() for f in chks]
    errs = [e for _, es in results for e in es]
    # a source that includes lds_dma.h but shows no load into LDS in its
    # assembly would otherwise pass unchecked
    errs += [f"{s}: no kernel with a load into LDS found in its assembly"
             for s, (c, _) in zip(checked_srcs, results) if not c]
    if errs:
        raise RuntimeError("static checks of the LDS-loading kernels failed:\n" + "\n".join(errs))
    if verbose:
        n = sum(len(c) for c, _ in results)
        print(f"static checks: {n} kernels in {', '.join(checked_srcs)} pass")
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
