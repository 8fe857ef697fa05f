"""Build the HIP library (gfx950) in-tree: chunkwise_causal_linear_amd/lib/libfla_linattn.so.

The fused chunk kernel is instantiated per (input dtype, key dimension) and the backward
kernels per (input dtype, contraction width) in separate objects compiled in parallel; the C ABI (include/fla_linattn.h) lives in fla_api.hip.
Usage: python -m chunkwise_causal_linear_amd.build [-j N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as fut
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "lib")
OBJDIR = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(LIBDIR, "libfla_linattn.so")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
    # keep the compiler from forming packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{os.path.join(ROOT, 'include')}",
]
DTYPES = [("bf16", 1), ("f32", 0)]
DKS = [16, 32, 64, 128, 256]
BWD_DYS = [64, 128, 256]


def _units():
    units = []
    for tname, flag in DTYPES:
        for dk in DKS:
            obj = os.path.join(OBJDIR, f"chunk_{tname}_{dk}.o")
            units.append((os.path.join(CSRC, "chunk_inst.hip"), obj,
                          [f"-DFLA_TIN_BF16={flag}", f"-DFLA_DK={dk}"]))
    for tname, flag in DTYPES:
        for dy in BWD_DYS:
            obj = os.path.join(OBJDIR, f"bwd_{tname}_{dy}.o")
            units.append((os.path.join(CSRC, "bwd_inst.hip"), obj,
                          [f"-DFLA_TIN_BF16={flag}", f"-DFLA_BWD_DY={dy}"]))
    units.append((os.path.join(CSRC, "gdn_inst.hip"), os.path.join(OBJDIR, "gdn_inst.o"), []))
    units.append((os.path.join(CSRC, "fla_api.hip"), os.path.join(OBJDIR, "fla_api.o"), []))
    units.append((os.path.join(CSRC, "probe.hip"), os.path.join(OBJDIR, "probe.o"), []))
    return units


def _deps_mtime(src: str) -> float:
    """Newest modification time of a unit's source and the local headers it includes
    (followed recursively through #include "...")."""
    seen, todo = set(), [os.path.abspath(src)]
    while todo:
        path = todo.pop()
        if path in seen or not os.path.exists(path):
            continue
        seen.add(path)
        with open(path) as f:
            for line in f:
                line = line.strip()
                if line.startswith("#include") and '"' in line:
                    name = line.split('"')[1]
                    todo.append(os.path.normpath(os.path.join(os.path.dirname(path), name)))
    return max(os.path.getmtime(p) for p in seen)


def _compile(unit, incremental: bool = False):
    src, obj, extra = unit
    if incremental and os.path.exists(obj) and os.path.getmtime(obj) > _deps_mtime(src):
        return obj
    tmp = obj + ".tmp.o"
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, obj)
    return obj


def build(jobs: int | None = None, verbose: bool = False, incremental: bool = False) -> str:
    """Compile every HIP translation unit for gfx950 and link the shared library.
    incremental=True keeps objects newer than their sources and headers."""
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    jobs = jobs or max(1, min(16, os.cpu_count() or 1))
    units = _units()
    with fut.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u, incremental), units))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=None)
    ap.add_argument("--incremental", action="store_true",
                    help="recompile only objects older than their sources or headers")
    args = ap.parse_args()
    build(args.j, verbose=True, incremental=args.incremental)
    sys.exit(0)
