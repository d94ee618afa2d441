"""Build libbsq.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m fp8_quantized_gemm_amd._build   (or __graft_entry__.build()).
Each translation unit is compiled to an object under _build/ in parallel,
then linked into fp8_quantized_gemm_amd/libbsq.so.  The measurement kernels
of the two GEMM routes' inner-loop ceilings go into a library of their own,
libbsq_ceiling.so, so the product ABI stays what include/bsq.h declares.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsq.so")
CEILING_LIB = os.path.join(PKG, "libbsq_ceiling.so")

SOURCES = ["bsq_api.cpp", "bsq_quantize.hip", "bsq_gemm.hip", "bsq_gemm_nvfp4.hip",
           "bsq_gemm_nvfp4_rx.hip", "bsq_gemm_mx_rx.hip"]
CEILING_SOURCES = ["route_a_ceiling.hip"]

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # bit-exact quantizers: IEEE FP32 ops, no fused multiply-add
    "-ffp-contract=off",
    # keep the compiler from forming packed FP32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libbsq")


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    return obj, "\n".join(warn)


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(out)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        results = list(ex.map(_compile, srcs))
    for (o, w), s in zip(results, srcs):
        if w and verbose:
            print(f"[bsq build] {s}:\n{w}", file=sys.stderr)
    objs = dict(zip(srcs, (o for o, _ in results)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in CEILING_SOURCES], CEILING_LIB)
    if verbose:
        print(f"[bsq build] wrote {LIB} and {CEILING_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
