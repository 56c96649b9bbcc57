"""Build libctopk.so in-tree with hipcc for gfx950.

Usage: python -m certified_top_sparse_amd.build   (or call build())

Each source compiles to its own object in parallel (the kernels of one
translation unit never call into another, so no relocatable device code is
needed), then hipcc links the objects into the shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libctopk.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "score_scan.hip", "select.hip", "bound.hip", "vsum.hip", "encoder.hip",
           "k4.hip", "shortrow.hip"]

COMPILE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-command-line-argument",
    # keep the compiler from emitting packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
LINK_FLAGS = ["--offload-arch=gfx950", "-shared", "-fPIC"]


def _filter(text: str):
    return [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libctopk.so (always recompiles)."""
    jobs = int(os.environ.get("MAX_JOBS", "0") or 0) or min(len(SOURCES), os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="ctopk_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]

        def compile_one(i):
            cmd = [HIPCC, *COMPILE_FLAGS, "-c", "-o", objs[i], os.path.join(CSRC, SOURCES[i])]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            return SOURCES[i], res.returncode, _filter(res.stdout + res.stderr)

        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(compile_one, range(len(SOURCES))))
        failed = [(s, msgs) for s, rc, msgs in results if rc != 0]
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(
                f"[{s}]\n" + "\n".join(msgs) for s, msgs in failed))
        if verbose:
            for s, _, msgs in results:
                if msgs:
                    print(f"[{s}]\n" + "\n".join(msgs))
        tmp = LIB + ".tmp"
        cmd = [HIPCC, *LINK_FLAGS, "-o", tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + "\n".join(_filter(res.stdout + res.stderr)))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
