"""MXFP4 and bf16 number formats: Python access to the C++ oracle's
definitions (oracle/moe_oracle.cpp).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package.  It shares no code with the HIP
path and never imports it.  This module only marshals arrays; every value
comes from the C++ oracle, except the byte shuffles pack_codes/unpack_codes
and the exact bit reinterpretation bf16_to_f64, which hold no rounding.

The pages name the format only as "MXFP4 weights" (VibeSys "Qwen3.5-397B on
4x MI300A" post, section "Goal"; its "Baseline" section: the fused HIP MoE
kernel dequantises MXFP4 in registers) and say nothing about its bits.  The
encoding is the OCP Microscaling (MX) v1.0 one: a block of 32 consecutive
elements along the reduction axis shares one E8M0 scale byte, and each
element is an FP4 E2M1 code (1 sign, 2 exponent, 1 mantissa bit, bias 1,
no Inf/NaN).  Two codes are packed per byte, element 2j in the low nibble.

Functions:
  e2m1_value(code)      closed form of one E2M1 code
  decode(packed, sc)    MXFP4 -> fp64, exact
  quantize(v)           fp64 values -> (packed, scales): OCP scale rule
                        (floor(log2 amax) - 2), nearest E2M1 value with ties
                        to the even code, saturating at 6, sign kept
  round_bf16(v)         fp64 -> nearest bf16 value (ties to even), one step
  bf16_bits(v)          fp64 -> bf16 bit patterns (uint16), via round_bf16
  bf16_to_f64(bits)     bf16 bit patterns -> fp64, exact
Pins: tests/test_oracle_mxfp4.py and tests/golden/mxfp4_blocks.json.
"""
from __future__ import annotations

import numpy as np

from ._lib import check, default_threads, lib, ptr

BLOCK = 32          # elements per scale block


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code s|ee|m: (-1)^s * 0.5*m for e == 0
    (subnormal) and (-1)^s * (1 + 0.5*m) * 2^(e-1) otherwise."""
    return lib().oracle_e2m1_value(int(code))


def __getattr__(name):
    """E2M1 (the 16 code values) and GRID (magnitudes of codes 0..7,
    ascending), built from the C++ oracle on first use."""
    if name == "E2M1":
        return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
    if name == "GRID":
        return np.array([e2m1_value(c) for c in range(8)], dtype=np.float64)
    raise AttributeError(name)


def e8m0_value(b):
    """Scale byte b -> 2^(b-127); byte 255 is NaN."""
    b = np.asarray(b, dtype=np.int64)
    f = np.vectorize(lambda v: lib().oracle_e8m0_value(int(v)), otypes=[np.float64])
    return f(b)[()] if b.ndim == 0 else f(b)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., n] -> codes uint8 [..., 2n]; element 2j is the low nibble."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = packed & 0x0F
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def decode(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 -> fp64: value = E2M1[code] * 2^(scale - 127).
    packed uint8 [..., K/2], scales uint8 [..., K/32] -> fp64 [..., K]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    K = packed.shape[-1] * 2
    rows = packed.size // max(packed.shape[-1], 1)
    assert scales.shape[-1] * BLOCK == K and scales.size == rows * (K // BLOCK)
    out = np.empty(packed.shape[:-1] + (K,), dtype=np.float64)
    check(lib().oracle_mxfp4_decode(ptr(packed), ptr(scales), rows, K, ptr(out)), "mxfp4 decode")
    return out


def quantize(v: np.ndarray, threads: int | None = None):
    """fp64 (or float32) [..., K] (K a multiple of 32) -> (packed uint8
    [..., K/2], scales uint8 [..., K/32]).

    Per block: amax = max |v|; X = floor(log2 amax) - 2, clamped to
    [-127, 127] (X = -127 for an all-zero block); scale byte X + 127.  Each
    v / 2^X is rounded to the nearest E2M1 magnitude, ties to the even code,
    saturating at 6; the sign bit of v is kept (so -0.0 and negatives that
    round to zero give code 0x8)."""
    v = np.asarray(v)
    f32 = v.dtype == np.float32
    v = np.ascontiguousarray(v, dtype=np.float32 if f32 else np.float64)
    K = v.shape[-1]
    assert K % BLOCK == 0
    rows = v.size // K
    packed = np.empty(v.shape[:-1] + (K // 2,), dtype=np.uint8)
    scales = np.empty(v.shape[:-1] + (K // BLOCK,), dtype=np.uint8)
    check(lib().oracle_mxfp4_quantize(ptr(v), int(f32), rows, K, ptr(packed), ptr(scales),
                                      threads or default_threads()), "mxfp4 quantize")
    return packed, scales


def round_bf16(v) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even, in one step
    (never through float32).  Results at or above 2^128 in magnitude
    overflow to +-inf."""
    a = np.array(v, dtype=np.float64, order="C")     # keeps 0-d input 0-d
    out = np.empty_like(a)
    lib().oracle_round_bf16_array(ptr(a), a.size, ptr(out))
    return out[()] if out.ndim == 0 else out


def bf16_bits(v) -> np.ndarray:
    """fp64 -> bf16 bit patterns (uint16), rounding as round_bf16."""
    a = np.array(v, dtype=np.float64, order="C")
    out = np.empty(a.shape, dtype=np.uint16)
    lib().oracle_bf16_bits_array(ptr(a), a.size, ptr(out))
    return out


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> their exact fp64 values (a bit reinterpretation)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
