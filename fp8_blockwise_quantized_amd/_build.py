"""Build libjetfp8.so (all HIP kernels + the C ABI) for gfx950 with hipcc.

Usage: python -m fp8_blockwise_quantized_amd._build
The library is written in-tree to fp8_blockwise_quantized_amd/lib/libjetfp8.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libjetfp8.so")
SOURCES = ["abi.hip", "quant.hip", "fused.hip", "kvcache.hip", "gemm.hip"]
# Roofline probes used by the benchmark only (include/jetprobe.h): a library of their own.
PROBE_LIB = os.path.join(LIBDIR, "libjetprobe.so")
PROBE_SOURCES = ["probes.hip"]
ARCH = "gfx950"

# No fast-math: the quantizers need IEEE division and FP32 denormals.
# Packed FP32 instructions are disabled for the device pass.  MFMA results are
# kept in VGPRs (the GEMMs fold every MFMA result with VALU FMAs; results in
# AGPRs would need one extra copy per element).
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    # never leave a library built from older sources behind a failed build
    for lib in (LIB, PROBE_LIB):
        if os.path.exists(lib):
            os.remove(lib)
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES) + len(PROBE_SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))
    for lib, lib_objs in ((LIB, objs[:len(SOURCES)]), (PROBE_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
