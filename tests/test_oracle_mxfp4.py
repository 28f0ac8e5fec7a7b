"""Pins of the oracle's number formats (oracle/mxfp4.py).

Each pin is something other than the oracle itself: the OCP MX table and
hand-worked blocks (tests/golden/mxfp4_blocks.json), a second formulation of
the rounding rule written here as thresholds, invariants of a nearest-value
quantiser, and torch's float32 -> bfloat16 conversion."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import mxfp4

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mxfp4_blocks.json")))


def test_e2m1_table_matches_spec():
    want = np.array(GOLD["e2m1_values"])
    got = np.array([mxfp4.e2m1_value(c) for c in range(16)])
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))   # codes 0 and 8 are +0 and -0


@pytest.mark.parametrize("case", GOLD["decode"])
def test_decode_worked(case):
    got = mxfp4.decode(np.array([[case["byte"]] * 16], np.uint8), np.array([[case["scale"]]], np.uint8))
    assert got[0, 0] == case["values"][0] and got[0, 1] == case["values"][1]


def test_decode_scale_nan_and_range():
    assert np.isnan(mxfp4.e8m0_value(255))
    assert mxfp4.e8m0_value(127) == 1.0 and mxfp4.e8m0_value(254) == 2.0 ** 127


@pytest.mark.parametrize("case", GOLD["quantize"])
def test_quantize_worked(case):
    blk = np.zeros(32)
    blk[:len(case["head"])] = case["head"]
    p, s = mxfp4.quantize(blk[None])
    assert int(s[0, 0]) == case["scale"]
    nb = len(case["bytes_head"])
    assert list(p[0, :nb]) == case["bytes_head"]
    assert np.all(p[0, nb:] == 0) or len(case["head"]) > 2 * nb
    dec = mxfp4.decode(p, s)[0]
    nd = len(case["decoded_head"])
    assert np.array_equal(dec[:nd], case["decoded_head"])
    assert np.array_equal(np.signbit(dec[:nd]), np.signbit(case["decoded_head"]))


def _threshold_code(a):
    """Second formulation of round-to-nearest-even onto E2M1 magnitudes:
    the midpoints between grid values, with the tie going to the even code."""
    a = np.asarray(a)
    code = np.full(a.shape, 7, np.uint8)
    # (upper bound, inclusive?, code): ties at 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5
    for bound, incl, c in [(5.0, True, 6), (3.5, False, 5), (2.5, True, 4), (1.75, False, 3),
                           (1.25, True, 2), (0.75, False, 1), (0.25, True, 0)]:
        m = (a <= bound) if incl else (a < bound)
        code = np.where(m, c, code)
    return code


def _all_bf16_below(limit):
    bits = np.arange(0, 0x8000, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    v = f[np.isfinite(f)].astype(np.float64)
    v = v[v < limit]
    return np.concatenate([v, -v])


@pytest.mark.parametrize("X", [-127, -126, -100, -7, -1, 0, 1, 60, 124])
def test_quantize_exhaustive_bf16_against_thresholds(X):
    """Every bf16 value below 8 * 2^X, in a block whose amax is 4 * 2^X
    (so the scale is X), quantises to the threshold rule's code."""
    v = _all_bf16_below(8.0) * 2.0 ** X
    n = v.size
    blocks = np.zeros((n, 32))
    blocks[:, 0] = 4.0 * 2.0 ** X
    blocks[:, 1] = v
    p, s = mxfp4.quantize(blocks)
    assert np.all(s[:, 0] == X + 127)
    codes = mxfp4.unpack_codes(p)[:, 1]
    want = _threshold_code(np.abs(v) / 2.0 ** X) | (np.signbit(v).astype(np.uint8) << 3)
    assert np.array_equal(codes, want)


def test_quantize_random_blocks_properties():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((4000, 64)) * np.exp2(rng.integers(-20, 20, (4000, 1)))
    p, s = mxfp4.quantize(v)
    d = mxfp4.decode(p, s)
    blocks = v.reshape(4000, 2, 32)
    amax = np.abs(blocks).max(-1)
    X = s.astype(np.int64) - 127
    # scale rule: 4 * 2^X <= amax < 8 * 2^X
    assert np.all(4.0 * np.exp2(X) <= amax) and np.all(amax < 8.0 * np.exp2(X))
    # error at most half a grid step (step 2 between 4 and 6, 1 between 2 and 4, ...) unless saturated
    scaled = np.abs(blocks) / np.exp2(X)[..., None]
    err = np.abs(d.reshape(4000, 2, 32) - blocks) / np.exp2(X)[..., None]
    step = np.where(scaled < 2, 0.5, np.where(scaled < 4, 1.0, 2.0))
    ok = (err <= step / 2 + 1e-12) | (scaled > 6)
    assert ok.all()
    # idempotent on its own output
    p2, s2 = mxfp4.quantize(d)
    assert np.array_equal(p2, p) and np.array_equal(s2, s)


def test_round_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = mxfp4.bf16_bits(f.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_bf16_single_rounding():
    # 1 + 2^-8 is a tie -> 1; 1 + 3*2^-8 is a tie -> 1 + 2^-6 (even); a tie plus a
    # tiny excess must round up, which float32-then-bf16 double rounding would lose.
    v = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -30, -0.0, 2.0 ** -133, 3 * 2.0 ** -134])
    got = mxfp4.bf16_to_f64(mxfp4.bf16_bits(v))
    assert list(got) == [1.0, 1 + 2 ** -6, 1 + 2 ** -7, 0.0, 2.0 ** -133, 2.0 ** -132]
    assert np.signbit(got[3])
    assert np.isinf(mxfp4.round_bf16(3.4e38)) and mxfp4.round_bf16(3.39e38) < np.inf


def test_pack_roundtrip():
    codes = np.arange(64, dtype=np.uint8).reshape(2, 32) % 16
    assert np.array_equal(mxfp4.unpack_codes(mxfp4.pack_codes(codes)), codes)
    assert mxfp4.pack_codes(np.array([[0x3, 0xA]], np.uint8))[0, 0] == 0xA3
