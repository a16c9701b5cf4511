"""Build libeta.so (HIP, gfx950) in the package directory with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libeta.so")
SOURCES = ["eta_summary.hip", "eta_screen.hip", "eta_attend.hip", "eta_calib.hip", "eta_prefill.hip", "eta_noalloc.hip", "eta_host.cpp"]
ARCH = os.environ.get("ETA_OFFLOAD_ARCH", "gfx950")

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# per-source flags: the calibration kernel's MFMA results go straight to
# vector registers (its binning reads every element; accumulation registers
# would need a copy of each first)
SOURCE_FLAGS = {"eta_calib.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


OBJ_DIR = os.path.join(HERE, "_build")  # objects of the last build (the sanitized build relinks them)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link libeta.so; always rebuilds."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="eta_build_") as tmp:
        objs = []
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [cc, *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), "-I", INCLUDE, *lang, "-c", os.path.join(CSRC, src),
                   "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs.pop(0), verbose)
        for p in procs:
            _wait(p, verbose)
        out_tmp = LIB + ".tmp"
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", out_tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode:
            raise RuntimeError("link failed:\n" + r.stdout)
        os.replace(out_tmp, LIB)
        os.makedirs(OBJ_DIR, exist_ok=True)
        for o in objs:
            shutil.copyfile(o, os.path.join(OBJ_DIR, os.path.basename(o)))
    return LIB


def _wait(item, verbose):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    if p.returncode:
        raise RuntimeError(f"hipcc failed on {src}:\n{text}")
    if verbose and text.strip():
        print(text, flush=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
