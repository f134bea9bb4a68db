"""Build libbi.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Every source is compiled with:
  * --offload-arch=gfx950, -O3;
  * -ffp-contract=off: the arithmetic of each output element is exactly what
    the source spells out (explicit fmaf where a fused multiply-add is meant);
  * -Xclang -target-feature -Xclang -packed-fp32-ops: no packed fp32 VALU
    instructions are generated;
  * no fast-math flags.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbi.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["api.cpp", "gemm_dispatch.hip", "gemm_bf16.hip", "gemm_kn.hip", "gemm_nvfp4.hip",
           "gemm_nvfp4raw.hip", "gemm_nvfp4a.hip", "gemm_skinny.hip", "gemm_pingpong.hip",
           "rmsnorm.hip", "nvfp4_quant.hip", "bmm.hip",
           "mla_decode.hip", "probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source for gfx950 and link libbi.so next to this file."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
