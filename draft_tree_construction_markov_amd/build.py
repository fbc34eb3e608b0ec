"""Build libpctree.so (HIP C++ for gfx950) in-tree with hipcc.

    python -m draft_tree_construction_markov_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpctree.so")
SOURCES = ["api.hip", "k_markov.hip",
           "k_markov_r2s.hip", "k_markov_r2d.hip", "k_markov_r4s.hip",
           "k_markov_r4d.hip", "k_markov_r8s.hip", "k_markov_r8d.hip",
           "k_markov_r16s.hip", "k_markov_r16d.hip", "k_select.hip",
           "k_verify.hip", "k_adaptive.hip", "profile.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    # packed fp32 VALU ops are disabled for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES
            if os.path.exists(os.path.join(CSRC, s))]


def _compile(src: str, obj: str, verbose: bool):
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source to an object file (in parallel), then link the
    shared library.  Always rebuilds."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), os.cpu_count() or 1, 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], verbose),
                    zip(srcs, objs)))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
           *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking libpctree failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
