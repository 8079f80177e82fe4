"""Build libsmoe.so in-tree with hipcc for gfx950.

    python -m sparse_mixture_experts_amd.build

Every ``csrc/*.hip`` file is compiled to an object under ``_build/`` and the objects
are linked into ``libsmoe.so`` next to this file.  Always recompiles.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libsmoe.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # Packed fp32 VALU ops stay off: hipcc must not form v_pk_{add,mul,fma}_f32.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build libsmoe.so")
    return path


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False, jobs: int | None = None, extra_flags=(), only=None) -> str:
    """Compile every csrc/*.hip (or, with ``only``, just the named sources, reusing the
    other objects from the last build) and link libsmoe.so.  Objects whose source no
    longer exists are deleted."""
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()

    def obj_of(src):
        return os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")

    wanted = {obj_of(s) for s in srcs}
    for stale in glob.glob(os.path.join(out_dir, "*.o")):
        if stale not in wanted:
            os.remove(stale)

    def compile_one(src):
        obj = obj_of(src)
        log = _run([cc, *HIP_FLAGS, *extra_flags, "-c", src, "-o", obj])
        if verbose and log.strip():
            print(log)
        return obj

    todo = srcs
    if only:
        names = {n if n.endswith(".hip") else n + ".hip" for n in only}
        todo = [s for s in srcs if os.path.basename(s) in names or not os.path.exists(obj_of(s))]
    jobs = jobs or min(16, os.cpu_count() or 4)
    with ThreadPoolExecutor(jobs) as pool:
        list(pool.map(compile_one, todo))
    objs = [obj_of(s) for s in srcs]
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    # python -m sparse_mixture_experts_amd.build [-v] [source.hip ...]: with source names,
    # recompile only those and relink.
    names = [a for a in sys.argv[1:] if a != "-v"]
    build(verbose="-v" in sys.argv, only=names or None)
