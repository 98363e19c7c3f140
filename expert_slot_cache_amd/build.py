"""Build libmoe_pool.so (HIP kernels + C-ABI runtime) for gfx950, in-tree.

    python -m expert_slot_cache_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_pool.so")

SOURCES = ["kernels.hip", "fill.hip", "policy.hip", "calibrate.hip", "moe_pool.cpp", "noalloc.cpp"]
ARCH = "gfx950"

# Every HIP compile disables packed fp32 instructions (v_pk_*_f32).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-parameter", "-Wno-unused-function"]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def build(verbose: bool = False, out: str = LIB, defines=(), objdir: str | None = None) -> str:
    objdir = objdir or os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmds.append([hipcc(), *HIP_FLAGS, *[f"-D{d}" for d in defines], "-I", INCLUDE, "-I", CSRC, *lang, "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    # the translation units are independent: compile them side by side
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        for f in [ex.submit(run, c) for c in cmds]:
            f.result()
    tmp = out + ".tmp"
    run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out

if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
