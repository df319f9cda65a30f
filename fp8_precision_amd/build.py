"""Build the gfx950 HIP library ``libfp8_precision.so`` in-tree with hipcc.

Usage: ``python fp8_precision_amd/build.py`` (or ``build()`` from Python).  Run it as
a script: importing the package loads the library this file builds.
Every call recompiles.  Compilation runs on the CPU; no GPU is needed.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfp8_precision.so")
SOURCES = ["quant.hip", "swiglu.hip", "gemm.hip", "copy.hip", "api.cpp"]
ARCH = "gfx950"

# Packed fp32 VALU instructions are kept out of the code object on purpose, and
# no multiply-add is contracted into an FMA: every fp32 step of the
# definitions (the SwiGLU tables, scales, encoders) is one IEEE operation.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}", f"-I{OBJDIR}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the FP8 library needs ROCm's hipcc to build")


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    # the SwiGLU tables swiglu.hip compiles in (silu_tables.inc)
    res = subprocess.run([sys.executable, os.path.join(CSRC, "gen_silu_tables.py"), OBJDIR],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gen_silu_tables.py failed:\n{res.stdout}\n{res.stderr}")
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
