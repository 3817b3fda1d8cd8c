"""Builds libdreamer.so (HIP, gfx950) in-tree with hipcc.

    python -m depth_recurrent_layer_amd.build        (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdreamer.so")
SOURCES = ["gemm.hip", "attn.hip", "route.hip", "expert_ffn.hip", "moe.hip", "usage.hip",
           "noalloc.hip", "api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
        "-Wno-unused-function", "-Wno-unused-variable",
        # packed fp32 ops stay off (hand-written or compiler-made v_pk_* f32 forms)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(HERE, "..", "include"),
    ]


def _compile(src: str, build_dir: str) -> str:
    obj = os.path.join(build_dir, src.replace(".", "_") + ".o")
    cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l).strip()
    if warn:
        sys.stderr.write(warn + "\n")
    return obj


def build(verbose: bool = True) -> str:
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
