"""Build libsanta.so in-tree with hipcc for gfx950.

    python -m sampled_sparse_decode_amd.build

compiles csrc/*.hip and csrc/*.cpp into sampled_sparse_decode_amd/libsanta.so.
Every invocation recompiles. Kernels are built for gfx950 only; packed FP32
instructions are disabled for device code.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libsanta.so")
ARCH = "gfx950"

SOURCES = ["santa_api.cpp", "reps.hip", "select.hip", "gather.hip", "pack.hip", "cluster.hip", "noalloc.hip",
           "value.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libsanta")
    return exe


def build(verbose=False, jobs=None):
    """Compile every source (in parallel, `jobs` at a time) and link
    libsanta.so; returns its path."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmds.append([hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)

    def compile_one(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(compile_one, c) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
