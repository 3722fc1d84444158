"""Host-sanitizer build of libmsr for the CPU boundary tests.

    python -m linear_recurrence_sequence_amd.build_sanitized

Compiles every HIP source with AddressSanitizer and UndefinedBehaviorSanitizer
on the host side only (the argument validation, workspace layout and
dispatch in msr_api.hip and the launchers; device code is built as usual),
links against the shared sanitizer runtime and writes
<repo>/_build_san/libmsr_san.so.  Run the ABI tests against it with

    LD_PRELOAD=$(python -m linear_recurrence_sequence_amd.build_sanitized --runtime) \\
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \\
    MSR_LIBRARY=<repo>/_build_san/libmsr_san.so python -m pytest tests/test_abi.py -q

(the binding loads the library named by MSR_LIBRARY when it is set).  The
tests there call only validation paths, so no GPU is needed.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

from .build import ARCH, CSRC, FLAGS, ROOT, hipcc, sources

OUT = os.path.join(ROOT, "_build_san")
LIB = os.path.join(OUT, "libmsr_san.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the HIP compiler."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    flags = [f if f != "-O3" else "-O1" for f in FLAGS] + ["-g"] + HOST_SAN
    r = subprocess.run([hipcc(), *flags, "-c", src, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, sources()))
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan",
           "-fsanitize=address,undefined", *objs, "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--runtime", action="store_true", help="print the sanitizer runtime to preload and exit")
    a = ap.parse_args()
    print(runtime() if a.runtime else build())
