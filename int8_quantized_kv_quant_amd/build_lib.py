"""Build libkvq.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m int8_quantized_kv_quant_amd.build_lib [--verbose]

Every HIP source is compiled for gfx950 only. Flags that matter for results:
  -fhip-fp32-correctly-rounded-divide-sqrt  the scale divisions (absmax / 127,
      the Q4_0 reciprocal 1 / d) must be IEEE correctly rounded;
  -Xclang -target-feature -Xclang -packed-fp32-ops  no packed fp32 VALU ops;
  -mllvm -amdgpu-mfma-vgpr-form  MFMA accumulators in VGPRs: the decode kernels
      scale MFMA results with VALU ops, and AGPR-resident accumulators cost a
      copy per element each time.
No fast-math flag is used anywhere.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvq.so")

SOURCES = ["kvq_host.cpp", "kvq_append.hip", "kvq_decode.hip", "kvq_decode_q4.hip", "kvq_reduce.hip", "kvq_chunk.hip",
           "kvq_chunk_q4.hip", "kvq_blob.hip", "kvq_stream.hip", "kvq_static.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
          "-I" + os.path.join(ROOT, "include")]
HIP_FLAGS = ["--offload-arch=gfx950", "-fno-gpu-rdc",
             "-fhip-fp32-correctly-rounded-divide-sqrt",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkvq)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON]
    if src.endswith(".hip"):
        cmd += HIP_FLAGS
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libkvq.so next to this file. Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libkvq.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
