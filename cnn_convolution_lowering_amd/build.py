"""Build the HIP library libconvlower.so in-tree for gfx950 (hipcc)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libconvlower.so")
SOURCES = [os.path.join(CSRC, f) for f in
           ("convlower.hip", "contract_f32.hip", "contract_f16.hip", "contract_bf16.hip")]
# The peak microbenchmarks (include/convpeak.h): a library of their own, so
# that nothing on the convolution path links them.
PEAK_LIB = os.path.join(PKG, "libconvpeak.so")
PEAK_SOURCE = os.path.join(CSRC, "peak.hip")

# Packed-fp32 instructions are kept out of every kernel: hipcc forms them from
# plain float code on its own, and they are not needed here.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the convolution library must be built with ROCm's hipcc")


def build_library(verbose: bool = False) -> str:
    """Compile each source to an object in parallel, then link the library."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    tag = "%d" % os.getpid()
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs = []
    peak_tmp = PEAK_LIB + ".tmp" + tag
    peak_cmd = [hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, PEAK_SOURCE, "-o", peak_tmp]
    if verbose:
        print(" ".join(peak_cmd), flush=True)
    peak_proc = subprocess.Popen(peak_cmd)
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(os.path.basename(src))[0] + "." + tag + ".o")
        cmd = [hipcc()] + compile_flags + ["-I", INCLUDE, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((subprocess.Popen(cmd), obj, cmd))
    failed = [cmd for proc, _, cmd in jobs if proc.wait() != 0]
    if peak_proc.wait() != 0:
        failed.append(peak_cmd)
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    os.replace(peak_tmp, PEAK_LIB)
    tmp = LIB + ".tmp" + tag
    cmd = [hipcc()] + HIPCC_FLAGS + [obj for _, obj, _ in jobs] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    for _, obj, _ in jobs:
        os.remove(obj)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
