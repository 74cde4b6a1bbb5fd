"""Builds libspecverify.so (gfx950 HIP kernels + the C ABI) in the package
directory.  Cross-compiles: no GPU is needed.

    python -m rejection_sampling_verifier_amd.build
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libspecverify.so")
ARCH = "gfx950"

SOURCES = ["sv_kernels.hip", "sv_produce.hip", "sv_api.cpp"]
DEPS = ["sv_internal.h", "sv_device.h"]


def hipcc():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def compile_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        # packed fp32 instructions stay off: hipcc forms them by itself otherwise
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{os.path.join(ROOT, 'include')}",
        f"-I{CSRC}",
    ]


def build(verbose=True, out=LIB, extra=()):
    """Compile every source and link the shared library (always rebuilds)."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [hipcc()] + compile_flags() + list(extra) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
