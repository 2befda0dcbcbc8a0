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


# device sources, compiled in parallel: the runtime, and the units that
# hold the kernel instances (mk_instances.h)
DEVICE_UNITS = ("mk_runtime", "mk_inst_wide", "mk_inst_gemv", "mk_inst_gemm", "mk_inst_all_p", "mk_inst_all_n")


def build(verbose: bool = True) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    host_obj = os.path.join(obj_dir, "mk_compile.o")
    cmds = [["g++", "-std=c++17", "-O2", "-fPIC", "-Wall", "-Wno-unused-function", "-c",
             os.path.join(CSRC, "mk_compile.cpp"), "-o", host_obj] + inc]
    dev_objs = []
    for unit in DEVICE_UNITS:
        obj = os.path.join(obj_dir, unit + ".o")
        dev_objs.append(obj)
        cmds.append([hipcc, "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
                     "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                     "-munsafe-fp-atomics", "-c", os.path.join(CSRC, unit + ".hip"), "-o", obj] + inc)
    procs = []
    for cmd in cmds:
        print("+", " ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd)))
    failed = [cmd for cmd, p in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", host_obj] + dev_objs + ["-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
