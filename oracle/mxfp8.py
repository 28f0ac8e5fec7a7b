"""MXFP8 (E4M3 elements) written out from its definition (fp64).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package.  It shares no code with the HIP
path and never imports it.

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

from . import mxfp4

BLOCK = 32          # elements per scale block
E4M3_EMAX = 8       # exponent of the largest E4M3 value (448 = 1.75 * 2^8)
NAN_CODE = 0x7F     # S.1111.111


def e4m3_value(code: int) -> float:
    """Value of an 8-bit E4M3 code s|eeee|mmm: (-1)^s * m/8 * 2^-6 for
    e == 0 (subnormal), NaN for e == 15 and m == 7, and
    (-1)^s * (1 + m/8) * 2^(e-7) otherwise."""
    s = (code >> 7) & 1
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


E4M3 = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# magnitudes of the finite non-negative codes 0..126, ascending with the code
GRID = E4M3[:NAN_CODE].copy()


def decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP8 -> fp64: value = E4M3[code] * 2^(scale - 127).
    codes uint8 [..., K], scales uint8 [..., K/32] -> fp64 [..., K]."""
    vals = E4M3[np.asarray(codes, dtype=np.uint8)]
    sc = mxfp4.e8m0_value(scales)
    return vals * np.repeat(sc, BLOCK, axis=-1)


def _nearest_code_magnitude(mag: np.ndarray) -> np.ndarray:
    """Code 0..126 of the GRID value nearest to mag (mag >= 0); on a tie the
    even code (mantissa bit 0) wins.  Values above 448 land on 448, the
    nearest grid value, so saturation needs no separate rule.  The two
    candidates are the grid neighbours of mag, found by binary search."""
    hi = np.clip(np.searchsorted(GRID, mag, side="left"), 1, len(GRID) - 1)
    lo = hi - 1
    d_lo = mag - GRID[lo]
    d_hi = GRID[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    return np.where(mag >= GRID[-1], len(GRID) - 1, code).astype(np.uint8)


def quantize(v: np.ndarray):
    """fp64 [..., K] (K a multiple of 32) -> (codes uint8 [..., K],
    scales uint8 [..., K/32]).

    Per block: amax = max |v|; X = floor(log2 amax) - 8, clamped to
    [-127, 127] (X = -127 for an all-zero block); scale byte X + 127.  Each
    v / 2^X is rounded to the nearest E4M3 magnitude, ties to the even code,
    saturating at 448; the sign bit of v is kept (so -0.0 and negatives that
    round to zero give code 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % BLOCK == 0
    blocks = v.reshape(*v.shape[:-1], K // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(amax)                 # amax = f * 2^ex, f in [0.5, 1)
    X = np.where(amax > 0, (ex - 1) - E4M3_EMAX, -127)
    X = np.clip(X, -127, 127)
    scaled = blocks / np.ldexp(1.0, X)[..., None]
    codes = _nearest_code_magnitude(np.abs(scaled))
    codes = codes | (np.signbit(scaled).astype(np.uint8) << 7)
    return codes.reshape(*v.shape[:-1], K), (X + 127).astype(np.uint8)
