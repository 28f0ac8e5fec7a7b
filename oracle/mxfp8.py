"""MXFP8 (E4M3 elements): Python access to the C++ oracle's definitions
(oracle/moe_oracle.cpp).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package.  It shares no code with the HIP
path and never imports it.  This module only marshals arrays.

The pages serve MoE models in MXFP8 as well as MXFP4 (MiniMax M3 on MI355X
post, section on its MI355X performance benchmarks: MXFP8 standard
inference next to MXFP4; the InferenceX Qwen3.5 post measures FP8 runs)
without giving the bits.  The encoding is the OCP Microscaling (MX) v1.0 one: 32 consecutive
elements along the reduction axis share one E8M0 scale byte (2^(b-127)),
and each element is one byte of FP8 E4M3: 1 sign, 4 exponent, 3 mantissa
bits, bias 7, no infinities, S.1111.111 = NaN, largest magnitude
1.75 * 2^8 = 448, subnormals m/8 * 2^-6.

Functions:
  e4m3_value(code)      closed form of one E4M3 code
  decode(codes, sc)     MXFP8 -> fp64, exact
  quantize(v)           fp64 values -> (codes, scales): OCP scale rule
                        (floor(log2 amax) - 8), nearest E4M3 value with ties
                        to the even code, saturating at 448, sign kept
Pins: tests/test_oracle_mxfp8.py and tests/golden/mxfp8_blocks.json.
"""
from __future__ import annotations

import numpy as np

from ._lib import check, default_threads, lib, ptr

BLOCK = 32          # elements per scale block
NAN_CODE = 0x7F     # S.1111.111


def e4m3_value(code: int) -> float:
    """Value of an 8-bit E4M3 code s|eeee|mmm: (-1)^s * m/8 * 2^-6 for
    e == 0 (subnormal), NaN for e == 15 and m == 7, and
    (-1)^s * (1 + m/8) * 2^(e-7) otherwise."""
    return lib().oracle_e4m3_value(int(code))


def __getattr__(name):
    """E4M3 (the 256 code values) and GRID (magnitudes of the finite
    non-negative codes 0..126, ascending with the code), built from the C++
    oracle on first use."""
    if name == "E4M3":
        return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    if name == "GRID":
        return np.array([e4m3_value(c) for c in range(NAN_CODE)], dtype=np.float64)
    raise AttributeError(name)


def decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP8 -> fp64: value = E4M3[code] * 2^(scale - 127).
    codes uint8 [..., K], scales uint8 [..., K/32] -> fp64 [..., K]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    K = codes.shape[-1]
    rows = codes.size // max(K, 1)
    assert scales.shape[-1] * BLOCK == K and scales.size == rows * (K // BLOCK)
    out = np.empty(codes.shape, dtype=np.float64)
    check(lib().oracle_mxfp8_decode(ptr(codes), ptr(scales), rows, K, ptr(out)), "mxfp8 decode")
    return out


def quantize(v: np.ndarray, threads: int | None = None):
    """fp64 (or float32) [..., K] (K a multiple of 32) -> (codes uint8
    [..., K], scales uint8 [..., K/32]).

    Per block: amax = max |v|; X = floor(log2 amax) - 8, clamped to
    [-127, 127] (X = -127 for an all-zero block); scale byte X + 127.  Each
    v / 2^X is rounded to the nearest E4M3 magnitude, ties to the even code,
    saturating at 448; the sign bit of v is kept (so -0.0 and negatives that
    round to zero give code 0x80)."""
    v = np.asarray(v)
    f32 = v.dtype == np.float32
    v = np.ascontiguousarray(v, dtype=np.float32 if f32 else np.float64)
    K = v.shape[-1]
    assert K % BLOCK == 0
    rows = v.size // K
    codes = np.empty(v.shape, dtype=np.uint8)
    scales = np.empty(v.shape[:-1] + (K // BLOCK,), dtype=np.uint8)
    check(lib().oracle_mxfp8_quantize(ptr(v), int(f32), rows, K, ptr(codes), ptr(scales),
                                      threads or default_threads()), "mxfp8 quantize")
    return codes, scales
