"""Ahead-of-time build of libditattn.so for gfx950 (hipcc, in-tree).

Each HIP source is compiled to an object in parallel, then linked into
``dit_joint_self_amd/libditattn.so``.  The build always recompiles; callers
that only need the library load the existing file.
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
LIB = os.path.join(PKG, "libditattn.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["api.hip", "prepare_kv.hip", "attn_core.hip", "attn_core_fp8.hip", "lse_merge.hip", "mxfp4.hip", "dbcache.hip", "clock_probe.hip", "rope_tables.hip"]

# Packed-fp32 VALU forms are disabled for all device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library needs ROCm's hipcc to build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


# Debug variant: every attention kernel fills its LDS buffers with NaN bytes
# before its first tile copy (DIT_DEBUG_LDS_NAN), so a read of LDS that no copy
# wrote poisons the output; the GPU tests compare it with the normal build.
DEBUG_LDS_NAN_LIB = os.path.join(PKG, "libditattn_ldsnan.so")
DEBUG_LDS_NAN_SOURCES = ["attn_core.hip", "attn_core_fp8.hip"]


def _build(lib_path: str, build_dir: str, extra: list, verbose: bool) -> str:
    cc = hipcc()
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = lib_path + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib_path)
    return lib_path


def build(verbose: bool = False, debug_lds_nan: bool = True) -> str:
    """Compile every HIP source for gfx950 and link libditattn.so (and, by
    default, the LDS-NaN debug variant); returns the main library's path."""
    _build(LIB, BUILD_DIR, [], verbose)
    if debug_lds_nan:
        _build(DEBUG_LDS_NAN_LIB, os.path.join(BUILD_DIR, "ldsnan"), ["-DDIT_DEBUG_LDS_NAN=1"], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
