"""Build and load the C++ oracle (oracle/moe_oracle.cpp) through ctypes.

TEST INFRASTRUCTURE.  The library is compiled with g++ (plain C++17, no GPU
headers) into oracle/_build/: libmoe_oracle.so for the Python wrappers and
moe_oracle, its command-line tool.  __graft_entry__.build() rebuilds both
every time; lib() builds them when they are missing or older than a source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libmoe_oracle.so")
CLI_PATH = os.path.join(BUILD_DIR, "moe_oracle")
SOURCES = [os.path.join(HERE, "moe_oracle.cpp")]
CLI_SOURCES = [os.path.join(HERE, "moe_oracle_cli.cpp")] + SOURCES
# x86-64-v3 (AVX2 + FMA) so the same build runs on any recent x86 host
CXXFLAGS = ["-O3", "-std=c++17", "-mavx2", "-mfma", "-fopenmp-simd", "-pthread", "-Wall",
            "-Wextra"]

_lock = threading.Lock()
_lib = None


def build() -> None:
    """Compile the shared library and the command-line tool (always)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    subprocess.run(["g++", *CXXFLAGS, "-fPIC", "-shared", *SOURCES, "-o", tmp], check=True)
    os.replace(tmp, LIB_PATH)
    tmp = CLI_PATH + ".tmp"
    subprocess.run(["g++", *CXXFLAGS, *CLI_SOURCES, "-o", tmp], check=True)
    os.replace(tmp, CLI_PATH)


def _declare(L):
    c = ctypes
    P = c.c_void_p
    i64, i32, dbl = c.c_int64, c.c_int32, c.c_double
    sig = {
        "oracle_default_threads": (c.c_int, []),
        "oracle_e2m1_value": (dbl, [c.c_int]),
        "oracle_e4m3_value": (dbl, [c.c_int]),
        "oracle_e8m0_value": (dbl, [c.c_int]),
        "oracle_round_bf16": (dbl, [dbl]),
        "oracle_bf16_bits": (c.c_uint16, [dbl]),
        "oracle_bf16_value": (dbl, [c.c_uint16]),
        "oracle_round_bf16_array": (None, [P, i64, P]),
        "oracle_bf16_bits_array": (None, [P, i64, P]),
        "oracle_mxfp4_quantize": (c.c_int, [P, c.c_int, i64, i64, P, P, c.c_int]),
        "oracle_mxfp8_quantize": (c.c_int, [P, c.c_int, i64, i64, P, P, c.c_int]),
        "oracle_mxfp4_decode": (c.c_int, [P, P, i64, i64, P]),
        "oracle_mxfp8_decode": (c.c_int, [P, P, i64, i64, P]),
        "oracle_route": (c.c_int, [P, P, i64, i32, i32, i32, i32, P, P]),
        "oracle_align": (c.c_int, [P, i64, i32, i32, P, P, P, P, P, i64, P]),
        "oracle_router_logits": (c.c_int, [P, P, i64, i64, i64, P, c.c_int]),
        "oracle_expert_mlp": (c.c_int, [P, i64, i64, i64, P, P, P, P, c.c_int, c.c_int, P, P,
                                        c.c_int]),
        "oracle_forward": (c.c_int, [P, P, P, P, P, P, P, i64, i64, i64, i32, i32, i32, c.c_int,
                                     c.c_int, i32, i32, P, i64, c.c_int, P, P, P, P, P, P]),
        "oracle_forward_from_h": (c.c_int, [P, P, P, P, P, i64, i64, i64, i32, i32, i32, c.c_int,
                                            c.c_int, i32, i32, c.c_int, P, P]),
        "oracle_residual_rmsnorm": (c.c_int, [P, i32, P, P, dbl, i64, i64, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def _stale() -> bool:
    """True when the library or the tool is missing or older than a source."""
    if not os.path.exists(LIB_PATH) or not os.path.exists(CLI_PATH):
        return True
    built = min(os.path.getmtime(LIB_PATH), os.path.getmtime(CLI_PATH))
    srcs = CLI_SOURCES + [os.path.join(HERE, "moe_oracle.h")]
    return any(os.path.getmtime(p) > built for p in srcs)


def lib():
    """The loaded oracle library (built first if it is missing or stale)."""
    global _lib
    with _lock:
        if _lib is None:
            if _stale():
                build()
            _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def default_threads() -> int:
    """Threads for the oracle's parallel loops: the CPUs of the affinity mask,
    at most 16 (one GPU's share of a shared host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def ptr(a) -> int | None:
    """Address of a numpy array's data (None for None)."""
    return None if a is None else a.ctypes.data


def check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"{what} rejected its arguments (status {rc})")
