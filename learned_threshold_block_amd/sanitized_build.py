"""Host-sanitizer build of libeta.so for the CPU ABI tests.

The host part of the library (eta_host.cpp: argument validation, workspace
layout, statistics read-back) is compiled with g++ under AddressSanitizer
and UndefinedBehaviorSanitizer (undefined behaviour traps, so no UB runtime
is needed) and linked with the kernel objects of the last regular build into
_build/libeta_sanitized.so. Load it with ETA_LIBRARY pointing at it and the
ASan runtime preloaded (asan_runtime()); the kernels themselves are the
regular gfx950 objects and are never launched by the CPU tests.
"""
from __future__ import annotations

import os
import subprocess
import sys

from . import build as B

SAN_LIB = os.path.join(B.OBJ_DIR, "libeta_sanitized.so")
HOST_FLAGS = ["-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
              "-fsanitize=address", "-fsanitize=undefined", "-fsanitize-undefined-trap-on-error"]


def asan_runtime() -> str:
    """Path of g++'s AddressSanitizer runtime (to put in LD_PRELOAD)."""
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def build_sanitized(verbose: bool = False) -> str:
    """Build _build/libeta_sanitized.so (runs the regular build first if its
    kernel objects are missing)."""
    kernels = [os.path.join(B.OBJ_DIR, s + ".o") for s in B.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in kernels):
        B.build(verbose=verbose)
    host_obj = os.path.join(B.OBJ_DIR, "eta_host_sanitized.o")
    cmd = ["g++", *HOST_FLAGS, "-I", "/opt/rocm/include", "-I", B.INCLUDE, "-c",
           os.path.join(B.CSRC, "eta_host.cpp"), "-o", host_obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    link = [B.hipcc(), "-shared", "-fPIC", f"--offload-arch={B.ARCH}", *kernels, host_obj, "-o", SAN_LIB]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    return SAN_LIB


if __name__ == "__main__":
    print(build_sanitized(verbose="-v" in sys.argv))
