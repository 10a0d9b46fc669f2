"""Builds libtq.so (host C++ + HIP kernels for gfx950) in-tree with hipcc.

Usage: python -m kv_cache_quantization_norm_amd.build   (or build_library()).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtq.so")
SOURCES = ["tq_host.cpp", "tq_kernels.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are disabled for all device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build_library(verbose: bool = False) -> str:
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(CSRC, src + ".o")
        cmd = [HIPCC, "-O3", "-std=c++17", "-fPIC", "-c", "-o", obj, "-I", INCLUDE, "-I", CSRC,
               "-Wall", "-Wno-unused-function"]
        if src.endswith(".hip"):
            cmd += DEVICE_FLAGS + ["-x", "hip"]
        cmd.append(path)
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "-o", tmp] + objs + DEVICE_FLAGS
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
