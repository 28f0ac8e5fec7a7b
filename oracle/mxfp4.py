"""MXFP4 and bf16 number formats, written out from their definitions (fp64).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package.  It shares no code with the HIP
path and never imports it.

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

BLOCK = 32          # elements per scale block
E2M1_EMAX = 2       # exponent of the largest E2M1 value (6 = 1.5 * 2^2)


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code s|ee|m: (-1)^s * 0.5*m for e == 0
    (subnormal) and (-1)^s * (1 + 0.5*m) * 2^(e-1) otherwise."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = 0.5 * m if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)
    return -mag if s else mag


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
# magnitudes of codes 0..7, ascending
GRID = E2M1[:8].copy()


def e8m0_value(b):
    """Scale byte b -> 2^(b-127); byte 255 is NaN."""
    b = np.asarray(b, dtype=np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


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
    vals = E2M1[unpack_codes(packed)]
    sc = e8m0_value(scales)
    return vals * np.repeat(sc, BLOCK, axis=-1)


def _nearest_code_magnitude(mag: np.ndarray) -> np.ndarray:
    """Index 0..7 of the GRID value nearest to mag; on a tie between two grid
    values the even index (mantissa bit 0) wins.  Values above 6 land on 6,
    which is the nearest grid value, so saturation needs no separate rule.
    Brute force over the 8 candidates, keeping the best so far (elementwise;
    evaluated in slices of 2^16 elements to stay in cache)."""
    flat = mag.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for lo in range(0, flat.size, 1 << 16):
        m = flat[lo:lo + (1 << 16)]
        best_code = np.zeros(m.shape, dtype=np.uint8)
        best_dist = np.abs(m - GRID[0])
        for c in range(1, 8):
            d = np.abs(m - GRID[c])
            take = (d < best_dist) | ((d == best_dist) & (c % 2 == 0))
            np.putmask(best_code, take, c)
            np.putmask(best_dist, take, d)
        out[lo:lo + (1 << 16)] = best_code
    return out.reshape(mag.shape)


def quantize(v: np.ndarray):
    """fp64 [..., K] (K a multiple of 32) -> (packed uint8 [..., K/2],
    scales uint8 [..., K/32]).

    Per block: amax = max |v|; X = floor(log2 amax) - 2, clamped to
    [-127, 127] (X = -127 for an all-zero block); scale byte X + 127.  Each
    v / 2^X is rounded to the nearest E2M1 magnitude, ties to the even code,
    saturating at 6; the sign bit of v is kept (so -0.0 and negatives that
    round to zero give code 0x8)."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % BLOCK == 0
    blocks = v.reshape(*v.shape[:-1], K // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(amax)                 # amax = f * 2^ex, f in [0.5, 1)
    X = np.where(amax > 0, (ex - 1) - E2M1_EMAX, -127)
    X = np.clip(X, -127, 127)
    scaled = blocks / np.ldexp(1.0, X)[..., None]
    codes = _nearest_code_magnitude(np.abs(scaled))
    codes = codes | (np.signbit(scaled).astype(np.uint8) << 3)
    codes = codes.reshape(*v.shape[:-1], K)
    return pack_codes(codes), (X + 127).astype(np.uint8)


def round_bf16(v) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even, in one step.
    bf16 keeps 8 significant bits and float32's exponent range; its spacing
    never drops below 2^-133 (the subnormal quantum).  Results at or above
    2^128 in magnitude overflow to +-inf."""
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(v)                    # |v| in [2^(ex-1), 2^ex)
    q = np.maximum(ex - 8, -133)           # exponent of the bf16 quantum
    r = np.ldexp(np.rint(np.ldexp(v, -q)), q)
    big = np.abs(r) >= 2.0 ** 128
    return np.where(big, np.copysign(np.inf, v), r)


def bf16_bits(v) -> np.ndarray:
    """fp64 -> bf16 bit patterns (uint16), rounding as round_bf16."""
    r = round_bf16(v).astype(np.float32)   # exact: r is bf16-representable
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
