"""Build the gfx950 shared library ``libmla_decode.so`` in-tree with hipcc,
and its debug build ``libmla_decode_debug.so``.

Usage: ``python -m paged_kv_mla_req_amd.build`` (or ``build()`` from Python).
Every source is compiled for gfx950 only; objects go to ``_build/`` next to
this file and the libraries are linked into the package directory.

The debug build is the same sources compiled with ``-DMLA_DEBUG`` plus
``debug_checks.hip``: the table builders and the decode check their
preconditions on the device (page-aligned slots, block-table entries inside
the table and the pool) and return MLA_ERR_PRECONDITION, synchronising the
stream to do so.  The kernels themselves are the release kernels.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla_decode.so")
DEBUG_LIB = os.path.join(PKG, "libmla_decode_debug.so")
SOURCES = ["abi.hip", "block_table.hip", "plan.hip", "decode.hip", "decode_q8.hip", "merge.hip",
           "append.hip", "noalloc.hip"]
DEBUG_SOURCES = SOURCES + ["debug_checks.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms stay disabled: the compiler would otherwise emit
# v_pk_{add,mul,fma}_f32 from ordinary float code.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# The decode kernels are compiled without NaN semantics, so that max() over
# scores is a plain v_max/v_max3 (no operand canonicalisation).  No NaN
# reaches it from the cache's unused slots: page tails are zero-filled, and
# masked scores are -inf, scaled by a factor kept above 0.
SOURCE_FLAGS = {"decode.hip": ["-fno-honor-nans"], "decode_q8.hip": ["-fno-honor-nans"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return res


def _build_one(sources, lib, extra, tag, verbose, jobs) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", tag + ".o"))
        cmd = [hipcc, *COMMON_FLAGS, *extra, *SOURCE_FLAGS.get(src, []), "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(sources)))) as ex:
        objs = list(ex.map(compile_one, sources))
    tmp = lib + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, jobs: int = 8, debug: bool = True) -> str:
    """Compile every source and link ``libmla_decode.so`` (and, with `debug`,
    ``libmla_decode_debug.so``); returns the release library's path."""
    path = _build_one(SOURCES, LIB, [], "", verbose, jobs)
    if debug:
        _build_one(DEBUG_SOURCES, DEBUG_LIB, ["-DMLA_DEBUG"], ".debug", verbose, jobs)
    return path


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
