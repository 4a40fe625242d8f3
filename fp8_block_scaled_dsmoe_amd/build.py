"""Build libdsmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python fp8_block_scaled_dsmoe_amd/build.py

Every source is compiled on each call (no staleness checks), in parallel,
then linked into fp8_block_scaled_dsmoe_amd/libdsmoe.so next to this file.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdsmoe.so")
SOURCES = ["abi.hip", "quant.hip", "granularity.hip", "serving.hip", "route.hip", "gemm.hip", "backward.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # exact IEEE semantics: no fast math, no contraction behind our back
    # (fused multiply-adds are written explicitly), correctly rounded
    # float32 division, no flushing of subnormals
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # keep packed-FP32 VALU instructions out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-Wall", "-Wno-unused-function",
    # the LDS-DMA helpers clobber M0 on purpose (they set it themselves)
    "-Wno-inline-asm",
]


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose: bool = True, jobs: int = 4) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for (o, err) in results:
            warn = "\n".join(l for l in err.splitlines() if "packed-fp32-ops" not in l and l.strip())
            if warn:
                print(warn, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def clean():
    shutil.rmtree(BUILD_DIR, ignore_errors=True)


if __name__ == "__main__":
    build()
