"""Host-sanitized build of libspecloss.so for the CPU tests of the C-ABI.

The host code (api.cpp: checks, plans, chunk policy, launch sequences) is
compiled with AddressSanitizer and UndefinedBehaviorSanitizer for the host
only; the kernels object of the regular build is linked in unchanged (no
sanitizer reaches device code).  The result lands in
lm_head_vocab_amd/_build/sanitize/libspecloss.so and is loaded by a Python
process started with the ASan runtime preloaded (see runtime_env).

Usage: python -m lm_head_vocab_amd.build_sanitized
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

from lm_head_vocab_amd import build as B

OUT_DIR = os.path.join(B.BUILD, "sanitize")
LIB = os.path.join(OUT_DIR, "libspecloss.so")
# each sanitizer flag is bound to the host compilation
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """The clang ASan runtime of the ROCm toolchain (preloaded into Python)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def runtime_env() -> dict:
    """Environment for a Python process that loads the sanitized library."""
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime()
    # the interpreter itself is not instrumented: its allocations at exit are
    # not leaks of the library
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["SPECLOSS_LIBRARY"] = LIB
    return env


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    kobj = os.path.join(B.BUILD, "kernels.hip.o")
    if not os.path.exists(kobj):
        B.build()
    aobj = os.path.join(OUT_DIR, "api.cpp.o")
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", *B.COMMON, *HOST_SAN, "-c",
           os.path.join(B.CSRC, "api.cpp"), "-o", aobj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", aobj,
           kobj, "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
