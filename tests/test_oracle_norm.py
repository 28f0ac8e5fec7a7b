"""Pins of the oracle's residual add + RMSNorm (oracle.moe.residual_rmsnorm):
the step after the layer in a tensor-parallel decode, where the ranks'
partial outputs are summed, the residual stream added and the sum
normalised (VibeSys "Qwen3.5-397B on 4x MI300A" post, section
"Communication and concurrency": the all-reduce fused with the residual add
and RMSNorm).  RMSNorm is taken in its textbook form
y = h / sqrt(mean(h^2) + eps) * gamma.

Each pin fixes a different part: the hand-worked fixture (sum, residual, bf16
rounding of h before the norm, per-column gamma, eps), closed forms (a
constant row normalises to its sign: catches a missing sqrt or a sum instead
of a mean), scale invariance by powers of two, and the plain cases G = 1 and
no residual.
"""
import json
import os

import numpy as np
import pytest

from oracle import moe, mxfp4

HERE = os.path.dirname(os.path.abspath(__file__))


def _bits(v):
    return mxfp4.bf16_bits(np.asarray(v, dtype=np.float64))


def _vals(b):
    return mxfp4.bf16_to_f64(np.asarray(b, dtype=np.uint16))


def test_golden_worked_rows():
    d = json.load(open(os.path.join(HERE, "golden", "residual_rmsnorm.json")))
    gamma = _bits(d["gamma"])
    for c in d["cases"]:
        h, y, rstd = moe.residual_rmsnorm(_bits(c["partials"]), _bits(c["residual"]), gamma,
                                          c["eps"])
        assert np.array_equal(_vals(h), np.array(c["h"]))
        assert np.allclose(rstd, c["rstd"], rtol=1e-15, atol=0)
        assert np.array_equal(_vals(y), np.array(c["y"]))


@pytest.mark.parametrize("c", [0.75, -3.0, 2.0 ** -6, 448.0])
def test_constant_row_normalises_to_its_sign(c):
    H = 64
    p = _bits(np.full((1, 1, H), c))
    h, y, rstd = moe.residual_rmsnorm(p, None, _bits(np.ones(H)), 0.0)
    assert np.array_equal(_vals(h), np.full((1, H), c))
    assert rstd[0] == pytest.approx(1.0 / abs(c), rel=1e-15)
    assert np.array_equal(_vals(y), np.full((1, H), np.sign(c)))


def test_power_of_two_scale_invariance():
    rng = np.random.default_rng(5)
    G, T, H = 3, 4, 96
    p = _vals(_bits(rng.standard_normal((G, T, H))))
    r = _vals(_bits(rng.standard_normal((T, H))))
    g = _bits(rng.uniform(0.5, 1.5, H))
    h1, y1, rs1 = moe.residual_rmsnorm(_bits(p), _bits(r), g, 0.0)
    h2, y2, rs2 = moe.residual_rmsnorm(_bits(p * 8.0), _bits(r * 8.0), g, 0.0)
    assert np.array_equal(_vals(h2), _vals(h1) * 8.0)
    assert np.allclose(rs2 * 8.0, rs1, rtol=1e-15)
    assert np.array_equal(y1, y2)


def test_single_partial_without_residual_is_plain_rmsnorm():
    rng = np.random.default_rng(6)
    T, H = 5, 128
    x = _vals(_bits(rng.standard_normal((T, H))))
    g = _vals(_bits(rng.uniform(0.5, 1.5, H)))
    eps = 1e-6
    h, y, rstd = moe.residual_rmsnorm(_bits(x[None]), None, _bits(g), eps)
    assert np.array_equal(_vals(h), x)
    want = 1.0 / np.sqrt(np.mean(x * x, axis=1) + eps)
    assert np.allclose(rstd, want, rtol=1e-14)
    assert np.array_equal(y, _bits(x * want[:, None] * g[None, :]))
    # y has unit RMS up to bf16 rounding when gamma = 1
    _, y1, _ = moe.residual_rmsnorm(_bits(x[None]), None, _bits(np.ones(H)), 0.0)
    assert np.sqrt(np.mean(_vals(y1) ** 2, axis=1)) == pytest.approx(np.ones(T), abs=4e-3)


def test_partials_and_residual_all_enter_the_sum():
    rng = np.random.default_rng(7)
    G, T, H = 4, 3, 32
    p = _vals(_bits(rng.standard_normal((G, T, H))))
    r = _vals(_bits(rng.standard_normal((T, H))))
    g = _bits(np.ones(H))
    h, _, _ = moe.residual_rmsnorm(_bits(p), _bits(r), g, 1e-6)
    assert np.array_equal(h, _bits(r + p.sum(axis=0)))
    # permuting the ranks changes nothing (fp64 sums of these bf16 values are exact)
    h2, _, _ = moe.residual_rmsnorm(_bits(p[::-1]), _bits(r), g, 1e-6)
    assert np.array_equal(h, h2)


def test_bad_arguments_are_rejected():
    p = _bits(np.ones((1, 2, 8)))
    g = _bits(np.ones(8))
    with pytest.raises(ValueError):
        moe.residual_rmsnorm(p, None, g, -1.0)
