"""Build the gfx950 shared library ``libmamba3_ssm.so`` in-tree with hipcc
(and ``libm3_floor.so``, the memory-floor probes that bench.py times).

Every HIP translation unit is compiled for gfx950 only, with packed-fp32 VALU
instructions disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``);
the objects go to ``_build/`` and are linked next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmamba3_ssm.so")
# memory-floor probes timed by bench.py --only floor (not part of the library)
FLOOR_LIB = os.path.join(HERE, "libm3_floor.so")
FLOOR_SOURCES = ["floor.hip"]
SOURCES = ["abi.cpp", "decode.hip", "rope.hip", "chunk.hip", "chunk_fast.hip", "chunk_subwalk.hip", "segments.hip", "backward.hip", "prologue.hip", "short_chunk.hip", "noalloc.cpp"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wno-unused-result", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source (always) and link the library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    fobjs = [_compile(src) for src in FLOOR_SOURCES]
    tmp = FLOOR_LIB + f".tmp{os.getpid()}"
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + fobjs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, FLOOR_LIB)
    if verbose:
        print(f"built {LIB} and {FLOOR_LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
