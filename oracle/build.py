"""Builds the CPU oracle libdreamer_ref.so in-tree with g++ (C++17, OpenMP).

    python -m oracle.build        (or build() from Python)

Test infrastructure: only the tests, the smoke check and the benchmark's CPU-baseline
leg load the library this builds."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dreamer_ref.cpp")
LIB = os.path.join(HERE, "libdreamer_ref.so")

# AVX2 + FMA (x86-64-v3) so the float64 dot products vectorise; no fast-math, so every
# operation is an IEEE float64 operation.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-mavx2", "-mfma", "-Wall",
         "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = True) -> str:
    tmp = LIB + ".tmp"
    cmd = ["g++"] + FLAGS + [SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
