"""Build of libhylra.so for gfx950 with hipcc (in-tree, next to this file)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhylra.so")
SOURCES = ["hylra_kernels.hip", "hylra_profile.hip", "hylra_offload.hip", "hylra_step.hip",
           "hylra_noalloc.hip", "hylra_api.cpp"]
ARCH = os.environ.get("HYLRA_OFFLOAD_ARCH", "gfx950")
COMPILE_TIMEOUT_S = 900  # a stuck compiler fails the build instead of hanging it

# Packed-fp32 VALU forms are disabled for every device compile.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in cand or os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile the HIP kernels and the C-ABI host code into libhylra.so."""
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-c",
               "-I" + os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]
        if src.endswith(".hip"):
            cmd += DEVICE_FLAGS
        else:
            cmd = [c for c in cmd if not c.startswith("--offload-arch")] + ["-x", "c++"]
        cmd += [path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd, timeout=COMPILE_TIMEOUT_S)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd, timeout=COMPILE_TIMEOUT_S)
    os.replace(tmp, LIB)
    for obj in objs:
        os.remove(obj)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
