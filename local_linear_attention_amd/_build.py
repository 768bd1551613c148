"""Builds liblla.so in-tree with hipcc for gfx950.

Each ``csrc/*.hip`` file compiles to an object in ``_build/`` in parallel; the objects
link into ``local_linear_attention_amd/liblla.so``.  Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblla.so")

ARCH = "gfx950"
# Packed fp32 VALU ops are switched off for all device code.
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-file flags: MFMA accumulators in architectural VGPRs.  The d = 128 kernels run one wave
# per SIMD with most of the register file in accumulators (the AGPR form made the register
# allocator shuffle accumulators between AGPRs inside the MFMA loop, which halved the
# matrix-core rate of a single wave).
FILE_FLAGS = {
    "lla_fast128.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
    # d = 64: the row-max kernel otherwise keeps its score accumulators in AGPRs and copies
    # them out every tile (0.057 -> 0.050 ms at d24); the other kernels are unchanged.
    "lla_fast.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        extra = FILE_FLAGS.get(os.path.basename(src), [])
        cmd = [cc, *HIPFLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
        if verbose and (res.stdout or res.stderr):
            print(res.stdout + res.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
