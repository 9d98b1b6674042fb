"""Build the HIP library ``libflashmask.so`` in-tree for gfx950 with hipcc.

Every HIP source is compiled with packed-fp32 instruction selection disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); nothing else is configurable.
``--stamps`` builds the debug variant ``libflashmask_stamps.so`` instead: the same sources with
FM_WG_STAMPS defined, whose attention kernels also record a per-workgroup timeline
(``include/flashmask_debug.h``, read by ``python -m mask_aware_flashattention_amd.wg_timeline``).
Usage: ``python -m mask_aware_flashattention_amd.build [--stamps]`` (``__graft_entry__.build()``
builds both).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libflashmask.so")
LIB_STAMPS = os.path.join(PKG, "libflashmask_stamps.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "mask_kernels.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_bwd_dq.hip",
           "noalloc.hip"]
# Per-source code-generation options (none at present).
EXTRA = {}
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]


def _hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; a ROCm toolchain is required to build the library")
    return exe


def _compile(src: str, verbose: bool, build_dir: str, defines: list) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *defines, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False, stamps: bool = False) -> str:
    """Compile every source and link the shared library (the debug variant with the workgroup
    timeline when ``stamps``); returns its path."""
    build_dir = os.path.join(BUILD_DIR, "stamps") if stamps else BUILD_DIR
    defines = ["-DFM_WG_STAMPS"] if stamps else []
    lib = LIB_STAMPS if stamps else LIB
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, defines), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, stamps="--stamps" in sys.argv[1:]))
