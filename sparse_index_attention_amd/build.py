"""Build libsia.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m sparse_index_attention_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsia.so")
SOURCES = ["indexer.hip", "indexer_bf16.hip", "topk.hip", "topk_pages.hip", "index_topk.hip", "quantize.hip", "sparse_mla.hip", "noalloc.hip", "sia_api.cpp"]
# per-source extra flags (none needed at present)
SOURCE_FLAGS = {}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; libsia needs the ROCm toolchain")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("libsia build failed:\n" + r.stderr[-8000:])
    if verbose:
        lines = [ln for ln in r.stderr.splitlines() if ln.strip() and "packed-fp32" not in ln]
        if lines:
            print("\n".join(lines[-40:]))


def build(verbose: bool = False, extra_flags=None, jobs: int = 4) -> str:
    """Compile every source and link libsia.so; returns its path.  Always rebuilds."""
    from concurrent.futures import ThreadPoolExecutor
    common = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
              # no packed-fp32 instructions (v_pk_{add,mul,fma}_f32)
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]
    common += list(extra_flags or [])
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(bdir, src + ".o")
        _run(common + SOURCE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    out_tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out_tmp] + objs, verbose)
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
