"""Build libmoe.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python fine_grained_mixture_router_amd/build.py
    python fine_grained_mixture_router_amd/build.py --phase

--phase builds a separate measurement copy, libmoe_phase.so (objects in
_build/phase), with -DMOE_PHASE_STAMPS: per-tile timestamps of the
many-rows GEMM tiles, read by phase_timing.py.  libmoe.so is not touched.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed fp32 instructions stay off in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, obj_dir: str = OBJ, defines=()) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *defines, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


PHASE_DIR = os.path.join(OBJ, "phase")
PHASE_LIB = os.path.join(HERE, "libmoe_phase.so")


def build(verbose: bool = False, phase: bool = False) -> str:
    obj_dir = PHASE_DIR if phase else OBJ
    lib = PHASE_LIB if phase else LIB
    defines = ("-DMOE_PHASE_STAMPS",) if phase else ()
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, obj_dir, defines), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True, phase="--phase" in sys.argv[1:])
    sys.exit(0)
