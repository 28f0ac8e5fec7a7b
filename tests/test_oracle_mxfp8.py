"""Pins of the oracle's MXFP8 format (oracle/mxfp8.py).

Each pin is something other than the oracle itself: torch's own E4M3
(float8_e4m3fn) decoding and rounding, hand-worked blocks
(tests/golden/mxfp8_blocks.json), a brute-force nearest-value search written
here, and invariants of a nearest-value quantiser."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import mxfp8

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mxfp8_blocks.json")))


def _torch_e4m3(codes):
    """Decode bytes with torch's float8_e4m3fn (a library definition of E4M3)."""
    t = torch.tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_e4m3_worked_values():
    for code, value, _ in GOLD["e4m3_values"]:
        got = mxfp8.e4m3_value(code)
        assert got == value and np.signbit(got) == np.signbit(value), code
    for code in GOLD["nan_codes"]:
        assert np.isnan(mxfp8.e4m3_value(code))


def test_e4m3_table_matches_torch():
    want = _torch_e4m3(np.arange(256))
    got = mxfp8.E4M3
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    assert np.all(np.diff(mxfp8.GRID) > 0) and mxfp8.GRID[-1] == 448.0


def test_decode_applies_block_scale():
    codes = np.full((1, 64), 0x38, np.uint8)               # 1.0 everywhere
    codes[0, 33] = 0xC4                                    # -3.0 in the second block
    got = mxfp8.decode(codes, np.array([[126, 130]], np.uint8))
    assert np.all(got[0, :32] == 0.5)
    assert got[0, 33] == -24.0 and got[0, 32] == 8.0


@pytest.mark.parametrize("case", GOLD["quantize"])
def test_quantize_worked(case):
    blk = np.zeros(32)
    blk[:len(case["head"])] = case["head"]
    q, s = mxfp8.quantize(blk[None])
    assert int(s[0, 0]) == case["scale"]
    n = len(case["codes_head"])
    assert list(q[0, :n]) == case["codes_head"]
    dec = mxfp8.decode(q, s)[0]
    nd = len(case["decoded_head"])
    assert np.array_equal(dec[:nd], case["decoded_head"])
    assert np.array_equal(np.signbit(dec[:nd]), np.signbit(case["decoded_head"]))


def _brute_codes(scaled):
    """Nearest of all 127 finite magnitudes by exhaustive search, ties to the
    even code; the sign bit of the input is kept."""
    grid = np.array([mxfp8.e4m3_value(c) for c in range(127)])
    mag = np.abs(scaled)[..., None]
    d = np.abs(mag - grid)
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(127), 1 << 20)
    even = np.where(cand % 2 == 0, cand, 1 << 20).min(axis=-1)
    code = np.where(even < (1 << 20), even, cand.min(axis=-1))
    return (code | (np.signbit(scaled).astype(np.int64) << 7)).astype(np.uint8)


def _scaled(v):
    blocks = v.reshape(*v.shape[:-1], -1, 32)
    amax = np.abs(blocks).max(axis=-1)
    X = np.clip(np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1))) - 8, -127), -127, 127)
    return (blocks / 2.0 ** X[..., None]).reshape(v.shape), X


def test_quantize_is_nearest_by_brute_force():
    rng = np.random.default_rng(11)
    v = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-12, 12, (64, 1)))
    # exact midpoints between neighbouring grid values (ties) and above 448
    mids = (mxfp8.GRID[:-1] + mxfp8.GRID[1:]) / 2
    v[0, :126] = mids[:126] * 2.0 ** -8 * np.sign(rng.standard_normal(126))
    v[0, 126:128] = [480 * 2.0 ** -8, -511 * 2.0 ** -8]
    q, s = mxfp8.quantize(v)
    sc, X = _scaled(v)
    assert np.array_equal(s, (X + 127).astype(np.uint8))
    assert np.array_equal(q, _brute_codes(sc))


def test_quantize_matches_torch_rounding_in_range():
    """torch's float32 -> float8_e4m3fn cast rounds to nearest, ties to even;
    on block-scaled values within +-448 it must give the oracle's codes."""
    rng = np.random.default_rng(12)
    v = rng.standard_normal((128, 512)).astype(np.float32).astype(np.float64)
    v[:, ::7] *= 1e-3                                      # subnormal-range elements
    q, s = mxfp8.quantize(v)
    sc, _ = _scaled(v)
    ok = np.abs(sc) <= 448
    t = torch.tensor(sc.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert ok.mean() > 0.99
    assert np.array_equal(q[ok], t[ok])


def test_quantize_invariants():
    rng = np.random.default_rng(13)
    v = rng.standard_normal((32, 128))
    q, s = mxfp8.quantize(v)
    d = mxfp8.decode(q, s)
    assert np.array_equal(mxfp8.quantize(d)[0], q)         # idempotent on grid values
    sc, X = _scaled(v)
    step = np.where(np.abs(sc) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(sc), 2.0 ** -6))) - 3),
                    2.0 ** -9)
    err = np.abs(d / np.repeat(2.0 ** X, 32, axis=-1) - sc)
    sat = np.abs(sc) > 448
    assert np.all(err[~sat] <= step[~sat] / 2)
    assert np.all(np.abs(d[sat]) == 448 * np.repeat(2.0 ** X, 32, axis=-1)[sat])
    z = mxfp8.quantize(np.array([[-0.0] + [0.0] * 31]))
    assert z[0][0, 0] == 0x80 and z[1][0, 0] == 0
