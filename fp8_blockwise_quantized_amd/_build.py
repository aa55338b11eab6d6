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
# The C ABI's host code (argument validation, dispatch, error text) built with
# AddressSanitizer and UndefinedBehaviorSanitizer, for the CPU validation tests
# (tests/test_abi_hostsan_cpu.py); the kernel objects are the ordinary ones.
HOSTSAN_LIB = os.path.join(LIBDIR, "libjetfp8_hostsan.so")
HOSTSAN_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer").split()
# Diagnostic build: the same library with the GEMM kernel's phase timing
# compiled in (include/jetphase.h), read by phase_timing.py.
PHASE_LIB = os.path.join(LIBDIR, "libjetfp8_phase.so")
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
    for lib in (LIB, PROBE_LIB, HOSTSAN_LIB, PHASE_LIB):
        if os.path.exists(lib):
            os.remove(lib)
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        extra = []
        if src.endswith("#phase"):
            src, extra = src[:-len("#phase")], ["-DJET_PHASE_TIMING=1"]
        obj = os.path.join(objdir, src.replace(".hip", "_phase.o" if extra else ".o"))
        cmd = [cc, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES) + len(PROBE_SOURCES) + 1) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES + ["gemm.hip#phase"]))
    phase_obj = objs.pop()
    # the ABI object again with host sanitizers, linked with the same kernel objects
    san_obj = os.path.join(objdir, "abi_hostsan.o")
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g", *HOSTSAN_FLAGS]
    r = subprocess.run([cc, *flags, "-c", os.path.join(CSRC, "abi.hip"), "-o", san_obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on abi.hip (host sanitizers):\n{r.stdout}\n{r.stderr}")
    san_objs = [san_obj if os.path.basename(o) == "abi.o" else o for o in objs[:len(SOURCES)]]
    phase_objs = [phase_obj if os.path.basename(o) == "gemm.o" else o for o in objs[:len(SOURCES)]]
    for lib, lib_objs in ((LIB, objs[:len(SOURCES)]), (PROBE_LIB, objs[len(SOURCES):]),
                          (HOSTSAN_LIB, san_objs), (PHASE_LIB, phase_objs)):
        tmp = lib + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)
    return LIB


def sanitizer_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (it carries the
    UndefinedBehaviorSanitizer handlers too); a process that loads the
    host-sanitized library preloads it."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    for cand in (clang, "/opt/rocm/llvm/bin/clang", shutil.which("clang") or ""):
        if cand and os.path.exists(cand):
            r = subprocess.run([cand, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                               text=True)
            path = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    raise RuntimeError("AddressSanitizer runtime not found")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
