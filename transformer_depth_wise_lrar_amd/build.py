"""Build liblrattnres.so for gfx950 with hipcc (in-tree, next to this file).

    python -m transformer_depth_wise_lrar_amd.build

Each HIP source compiles to an object in _build/, then the objects link into one shared
library. Packed-FP32 instruction selection is disabled for every device pass.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "liblrattnres.so")
SOURCES = ["lrar_api.hip", "lrar_read.hip", "lrar_tile.hip", "lrar_tile_online.hip",
           "lrar_tile_twopass.hip", "lrar_tile_merge.hip", "lrar_tile_merge_acc.hip",
           "lrar_tile_variants.hip", "lrar_stats.hip", "lrar_stats_tile.hip",
           "lrar_backward.hip", "lrar_backward_tile.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source for gfx950 and link liblrattnres.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
