"""Build libsala.so (HIP for gfx950) in-tree with hipcc.

Every source under csrc/ is compiled for --offload-arch=gfx950 into _build/ and linked into
hybrid_sparse_linear_causal_amd/libsala.so; csrc/peaks/peaks.hip (the measured-ceiling kernels
of bench.py) becomes libsala_peaks.so; libsala_asan.so is the same library with its host code
built with AddressSanitizer and UndefinedBehaviorSanitizer (for the argument-check tests on the
CPU). Packed-fp32 VALU instructions are disabled for
the device code (-Xclang -target-feature -Xclang -packed-fp32-ops).

    python -m hybrid_sparse_linear_causal_amd.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsala.so")

ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Wno-unused-result"]


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libsala needs the ROCm toolchain to build")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose=False, jobs=8):
    """Compile every source and link libsala.so. Always rebuilds. Returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        cmd = [hipcc, *COMMON, *DEVICE_FLAGS, "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd = [hipcc, *COMMON, "-x", "hip", *DEVICE_FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose and errs.strip():
            print(errs, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    r = subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    build_peaks(hipcc)
    build_asan(jobs)
    return LIB


ASAN_BUILD = os.path.join(PKG, "_build_asan")
ASAN_LIB = os.path.join(PKG, "libsala_asan.so")
# host code instrumented with AddressSanitizer and UndefinedBehaviorSanitizer (the device code is
# built as usual); for the argument-checking tests on the CPU, run with the clang ASan runtime
# preloaded (asan_runtime())
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def asan_runtime():
    r = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if path and os.path.exists(path) else None


def build_asan(jobs=8):
    """libsala_asan.so: the library with sanitizer-instrumented host code."""
    hipcc = _hipcc()
    os.makedirs(ASAN_BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(ASAN_BUILD, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        r = subprocess.run([hipcc, *COMMON, *lang, *DEVICE_FLAGS, *ASAN_FLAGS, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (sanitized host) failed for {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, sources()))
    tmp = ASAN_LIB + ".tmp"
    r = subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", *ASAN_FLAGS, "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (sanitized host) failed:\n{r.stderr}")
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


PEAKS_SRC = os.path.join(CSRC, "peaks", "peaks.hip")
PEAKS_LIB = os.path.join(PKG, "libsala_peaks.so")


def build_peaks(hipcc=None):
    """The measured-ceiling kernels bench.py uses (libsala_peaks.so; not part of libsala)."""
    hipcc = hipcc or _hipcc()
    tmp = PEAKS_LIB + ".tmp"
    r = subprocess.run([hipcc, *COMMON, *DEVICE_FLAGS, "-shared", PEAKS_SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PEAKS_SRC}:\n{r.stderr}")
    os.replace(tmp, PEAKS_LIB)
    return PEAKS_LIB


if __name__ == "__main__":
    print(build(verbose=True))
