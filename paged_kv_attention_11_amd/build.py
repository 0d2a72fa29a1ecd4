"""Build libpagedattn.so (gfx950) in-tree with hipcc.

    python -m paged_kv_attention_11_amd.build [--verbose]

Each csrc/*.hip file is compiled separately (in parallel) and linked into one
shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
BUILD = PKG / "_build"
LIB = PKG / "libpagedattn.so"
INCLUDE = PKG.parent / "include"
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unknown-pragmas",
    # packed fp32 VALU forms are kept out of all generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(
        line for line in r.stdout.splitlines()
        if "packed-fp32-ops' is not a recognized feature" not in line
    )
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int | None = None) -> Path:
    """Compile every HIP source and link the shared library; returns its path."""
    BUILD.mkdir(exist_ok=True)
    srcs = sorted(CSRC.glob("*.hip"))
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    objs = [BUILD / (s.stem + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    cmds = [[HIPCC, *COMMON, "-I", str(INCLUDE), "-c", str(s), "-o", str(o)] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB.with_suffix(".so.tmp")
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    p = build(verbose="--verbose" in sys.argv)
    print(p)
