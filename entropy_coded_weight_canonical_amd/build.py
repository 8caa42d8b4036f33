"""Compile the library (HIP kernels for gfx950 + host code) into ``libentro.so``.

    python -m entropy_coded_weight_canonical_amd.build

Always rebuilds.  The shared object lands next to this file so that it ships
with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libentro.so")
SOURCES = ["entro_decode.hip", "entro_rans.hip", "entro_lut.cpp", "entro_encode.cpp", "entro_rans.cpp"]
ARCH = os.environ.get("ENTRO_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    objs = []
    common = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(build_dir, src + ".o")
        if src.endswith(".hip"):
            cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                   "-c", path, "-o", obj] + common
        else:
            rocm_inc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
            cmd = [hipcc(), "-x", "c++", f"-I{rocm_inc}", "-D__HIP_PLATFORM_AMD__", "-c", path, "-o", obj] + common
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + ["-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
