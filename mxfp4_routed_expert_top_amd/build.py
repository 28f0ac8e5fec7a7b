"""Build libmoe_mxfp4.so (the C-ABI library and its HIP kernels) for gfx950.

usage: python -m mxfp4_routed_expert_top_amd.build [--debug | --all]
Compiles every csrc/*.hip and csrc/*.cpp with hipcc into
mxfp4_routed_expert_top_amd/libmoe_mxfp4.so, in the source tree; --debug
builds libmoe_mxfp4_debug.so instead (-DMOE_DEBUG: the kernels' bound
checks, see moe_debug_flags), --all both.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_mxfp4.so")
DEBUG_LIB = os.path.join(PKG, "libmoe_mxfp4_debug.so")
BUILD_DIR = os.path.join(PKG, "_build")
DEBUG_BUILD_DIR = os.path.join(PKG, "_build_debug")
ARCH = "gfx950"

# -packed-fp32-ops keeps hipcc from emitting packed fp32 VALU ops (v_pk_*_f32)
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(os.path.dirname(PKG), "include")]


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(DEBUG_BUILD_DIR if debug else BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *(["-DMOE_DEBUG"] if debug else []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


def _sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = True, debug: bool = False, both: bool = False) -> str:
    """Compile the library (debug: the MOE_DEBUG build; both: the two, their
    sources compiled side by side).  Returns the (last) library's path."""
    variants = [False, True] if both else [debug]
    for d in variants:
        os.makedirs(DEBUG_BUILD_DIR if d else BUILD_DIR, exist_ok=True)
    srcs = _sources()
    jobs = [(src, d) for d in variants for src in srcs]
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    for i, d in enumerate(variants):
        lib = DEBUG_LIB if d else LIB
        _link(objs[i * len(srcs):(i + 1) * len(srcs)], lib)
        if verbose:
            print(f"built {lib} from {len(srcs)} sources")
    return DEBUG_LIB if variants[-1] else LIB


if __name__ == "__main__":
    build(debug="--debug" in sys.argv, both="--all" in sys.argv)
