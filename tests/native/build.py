"""Compile the native C++ callers of include/pa.h (tests/native/decode_step and
prefill_step) with g++.

A plain host compiler, the header, libpa.so and the HIP runtime are all a native caller
needs; each program finds libpa.so through its rpath, so it runs from wherever the tree is.

    python -m tests.native.build
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PROGRAMS = ("decode_step", "prefill_step")
SRC = os.path.join(HERE, "decode_step.cpp")
EXE = os.path.join(HERE, "decode_step")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    """Compile and link every program (libpa.so must exist); returns the decode program's path."""
    cxx = shutil.which("g++")
    if cxx is None:
        raise RuntimeError("g++ not found")
    for name in PROGRAMS:
        exe = os.path.join(HERE, name)
        tmp = exe + ".tmp"
        cmd = [cxx, "-O2", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__",
               f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROCM, 'include')}",
               os.path.join(HERE, name + ".cpp"),
               f"-L{os.path.join(ROOT, 'paged_kv_cache_67_amd')}", "-lpa",
               f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64",
               "-Wl,-rpath,$ORIGIN/../../paged_kv_cache_67_amd",
               f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, exe)
        if verbose:
            print(f"built {exe}")
    return EXE

if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
