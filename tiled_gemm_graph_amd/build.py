"""Build libmk.so in-tree: the host compiler (C++17) and the gfx950 kernels.

    python -m tiled_gemm_graph_amd.build        (or: python tiled_gemm_graph_amd/build.py)
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
ARCH = os.environ.get("MK_OFFLOAD_ARCH", "gfx950")


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def build(verbose: bool = True) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    host_obj = os.path.join(obj_dir, "mk_compile.o")
    _run(["g++", "-std=c++17", "-O2", "-fPIC", "-Wall", "-Wno-unused-function", "-c",
          os.path.join(CSRC, "mk_compile.cpp"), "-o", host_obj] + inc)
    dev_obj = os.path.join(obj_dir, "mk_runtime.o")
    _run([hipcc, "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics", "-c", os.path.join(CSRC, "mk_runtime.hip"), "-o", dev_obj] + inc)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", host_obj, dev_obj, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
