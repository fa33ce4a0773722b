"""Build libdiffattn.so for gfx950 with hipcc (in-tree, next to this file).

    python -m differential_attention_v2_amd.build_lib [--verbose] [--resource-usage]

Objects go to ``_build/`` at the repository root; the shared library is written
to ``differential_attention_v2_amd/libdiffattn.so``.
"""
from __future__ import annotations

import argparse
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
LIB = os.path.join(PKG, "libdiffattn.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "prefill_bf16.hip", "decode_bf16.hip", "rows_f32.hip", "backward_bf16.hip", "proj_bf16.hip",
           "gemm_bf16.hip", "noalloc_scratch.hip"]
LIBS = []

# Packed-fp32 VALU instructions are kept out of every kernel; hipcc -O3 would
# otherwise form them from plain float code.
# MFMA results are selected into VGPRs (not AGPRs): the online-softmax rescale
# multiplies the accumulators with VALU ops, and AGPR accumulators made the
# compiler copy them between register files on every tile.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libdiffattn needs ROCm's hipcc to build")


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose and (r.stdout.strip() or r.stderr.strip()):
        print(r.stdout + r.stderr, flush=True)


def build(verbose: bool = False, resource_usage: bool = False, jobs: int = 8) -> str:
    """Compile every source for gfx950 and link libdiffattn.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([hipcc, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj], verbose or resource_usage)
        return obj

    with ThreadPoolExecutor(max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs, *LIBS], verbose)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true", help="print per-kernel register/LDS usage")
    args = ap.parse_args(argv)
    path = build(verbose=args.verbose, resource_usage=args.resource_usage)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
