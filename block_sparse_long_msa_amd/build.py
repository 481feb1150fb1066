"""Build libmsa.so and libmsa_debug.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m block_sparse_long_msa_amd.build [-v] [--release-only]
Every call recompiles; objects go to _build/ (release) and _build/debug/ at
the repository root and the shared libraries next to this file.  The debug
library is the same code built with -DMSA_DEBUG: its kernels count failed
gather bounds checks on the device (msa_debug_bounds_violations).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmsa.so")
DEBUG_LIB = os.path.join(PKG, "libmsa_debug.so")
ARCH = "gfx950"

# -packed-fp32-ops keeps the compiler from emitting packed fp32 VALU ops.
COMMON = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str, verbose: bool, debug: bool) -> str:
    obj = os.path.join(BUILD, "debug" if debug else "", os.path.basename(src) + ".o")
    cmd = ["hipcc", "-c", *COMMON, *(["-DMSA_DEBUG"] if debug else []), src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines()
                    if "packed-fp32-ops" not in line)   # host-pass notice, harmless
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = ["hipcc", "-shared", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, debug: bool = True) -> str:
    """Compile and link libmsa.so (and, with `debug`, libmsa_debug.so);
    returns the release library's path."""
    os.makedirs(os.path.join(BUILD, "debug"), exist_ok=True)
    srcs = sources()
    jobs = [(s, False) for s in srcs] + ([(s, True) for s in srcs] if debug else [])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    _link(objs[:len(srcs)], LIB, verbose)
    if debug:
        _link(objs[len(srcs):], DEBUG_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, debug="--release-only" not in sys.argv))
