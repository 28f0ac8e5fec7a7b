"""Pins of the oracle's layer (oracle/moe.py).

Hand-worked routing and grouping (tests/golden/route_align.json), brute force
on tiny inputs, a library softmax, the reduction of a one-expert layer to a
dense SwiGLU MLP computed by plain loops, the equivalence of a folded-in
shared expert with a separate dense MLP, and invariants (linearity in the
down-projection scale, token-permutation equivariance, expert relabelling)."""
import json
import math
import os

import numpy as np
import torch
import pytest
import scipy.special

import synth
from oracle import moe, mxfp4, mxfp8

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "route_align.json")))
E2M1_TABLE = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mxfp4_blocks.json")))["e2m1_values"]


@pytest.mark.parametrize("case", GOLD["route"])
def test_route_worked(case):
    ids, w = moe.route(np.array([case["logits"]], np.float32), None, case["K"], 0)
    assert list(ids[0]) == case["ids"]
    assert np.allclose(w[0], case["w"], atol=1e-7)


@pytest.mark.parametrize("case", GOLD["shared_gate"])
def test_shared_gate_worked(case):
    ids, w = moe.route(np.zeros((1, 4), np.float32), np.array([case["g"]], np.float32), 2, 1)
    assert ids[0, 2] == 4
    assert abs(w[0, 2] - case["w"]) < 1e-7


def test_route_brute_force_with_ties():
    for seed, (T, E, K) in enumerate([(50, 16, 4), (30, 33, 7), (20, 8, 8)]):
        l = synth.ties_logits(T, E, seed).numpy()
        ids, w = moe.route(l, None, K, 0)
        for t in range(T):
            order = sorted(range(E), key=lambda e: (-float(l[t, e]), e))[:K]
            assert list(ids[t]) == order
            top = [math.exp(float(l[t, e]) - float(l[t, order[0]])) for e in order]
            assert np.allclose(w[t], [x / sum(top) for x in top], rtol=0, atol=1e-7)


def test_route_weights_sum_to_one():
    rng = np.random.default_rng(1)
    l = rng.standard_normal((300, 512)).astype(np.float32)
    _, w = moe.route(l, None, 10, 0)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) < 1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)          # slots in descending weight


def test_route_full_softmax_is_library_softmax():
    rng = np.random.default_rng(2)
    l = rng.standard_normal((20, 12)).astype(np.float32)
    ids, w = moe.route(l, None, 12, 0, renormalize=False)
    ref = scipy.special.softmax(l.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(ref, ids, 1), atol=1e-7)


def test_align_worked():
    a = GOLD["align"]
    counts, offsets, srt, inv, tiles, n = moe.align(np.array(a["ids"]), a["Ep"], a["tile_m"])
    assert list(counts) == a["counts"] and list(offsets) == a["offsets"]
    assert list(srt) == a["sorted"] and tiles.tolist() == a["tiles"] and n == a["n_tiles"]
    assert np.array_equal(srt[inv], np.arange(6))


def test_align_brute_force():
    rng = np.random.default_rng(3)
    for T, Kp, Ep, tm in [(37, 3, 9, 4), (5, 2, 20, 32), (64, 11, 13, 32), (1, 1, 1, 32)]:
        ids = rng.integers(0, Ep, (T, Kp))
        counts, offsets, srt, inv, tiles, n = moe.align(ids, Ep, tm)
        flat = ids.reshape(-1).tolist()
        want_sorted, want_tiles = [], []
        for e in range(Ep):                       # counting sort by plain loops
            group = [a for a in range(len(flat)) if flat[a] == e]
            for s in range(0, len(group), tm):
                want_tiles.append([e, len(want_sorted) + s])
            want_sorted += group
            assert counts[e] == len(group)
        assert srt.tolist() == want_sorted and tiles.tolist() == want_tiles and n == len(want_tiles)
        assert offsets[-1] == T * Kp and np.all(np.diff(offsets) == counts)


def _make_weights(cfg, rng_seed=0):
    """Random MXFP4 weights for a small config, packed by the oracle."""
    w13 = [mxfp4.quantize(synth.expert_w13(cfg, e).double().numpy()) for e in range(cfg.Ep)]
    w2 = [mxfp4.quantize(synth.expert_w2(cfg, e).double().numpy()) for e in range(cfg.Ep)]
    return lambda e: (w13[e][0], w13[e][1], w2[e][0], w2[e][1])


def _inputs(cfg):
    x = synth.activations(cfg).view(__import__("torch").int16).numpy().view(np.uint16)
    l = synth.router_logits(cfg).numpy()
    g = synth.gate_logits(cfg)
    return x, l, (None if g is None else g.numpy())


def _decode_by_table(packed, scales):
    """Independent decode for the dense reduction test: table lookup from the
    golden E2M1 list and 2**(b - 127), element 2j from the low nibble."""
    rows, nb = packed.shape
    out = [[0.0] * (2 * nb) for _ in range(rows)]
    for r in range(rows):
        for j in range(nb):
            b = int(packed[r, j])
            sc = 2.0 ** (int(scales[r, (2 * j) // 32]) - 127)
            out[r][2 * j] = E2M1_TABLE[b & 15] * sc
            out[r][2 * j + 1] = E2M1_TABLE[b >> 4] * sc
    return out


def test_one_expert_reduces_to_dense_swiglu_mlp():
    """With y kept (the default) out_f64 is the dense MLP's output; with
    round_y each output is that value rounded to bf16."""
    cfg = synth.custom_config(T=3, H=64, I=32, E=1, K=1, shared=0)
    W = _make_weights(cfg)
    x, l, _ = _inputs(cfg)
    res = moe.forward(x, l, None, W, cfg.I, cfg.E, cfg.K, 0)
    res_r = moe.forward(x, l, None, W, cfg.I, cfg.E, cfg.K, 0, round_y=True)
    w13, w13s, w2, w2s = W(0)
    A = _decode_by_table(w13, w13s)        # [2I][H]
    B = _decode_by_table(w2, w2s)          # [H][I]
    xv = mxfp4.bf16_to_f64(x)
    for t in range(cfg.T):
        h = []
        for i in range(cfg.I):
            g = sum(A[i][k] * xv[t, k] for k in range(cfg.H))
            u = sum(A[cfg.I + i][k] * xv[t, k] for k in range(cfg.H))
            h.append(float(mxfp4.round_bf16(g / (1 + math.exp(-g)) * u)))
        for j in range(cfg.H):
            y = sum(B[j][i] * h[i] for i in range(cfg.I))
            assert abs(res["out_f64"][t, j] - y) <= 1e-12 * max(1.0, abs(y))
            yr = float(mxfp4.round_bf16(y))
            assert abs(res_r["out_f64"][t, j] - yr) <= 1e-12 * max(1.0, abs(yr))
    assert np.all(res["w"] == 1.0)


def _make_weights_mxfp8(cfg):
    """Random MXFP8 weights for a small config, packed by the oracle."""
    w13 = [mxfp8.quantize(synth.expert_w13(cfg, e).double().numpy()) for e in range(cfg.Ep)]
    w2 = [mxfp8.quantize(synth.expert_w2(cfg, e).double().numpy()) for e in range(cfg.Ep)]
    return lambda e: (w13[e][0], w13[e][1], w2[e][0], w2[e][1])


def _decode_e4m3_by_torch(codes, scales):
    """Independent MXFP8 decode: torch's float8_e4m3fn values times 2^(b-127)."""
    v = torch.tensor(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return (v * np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=-1)).tolist()


def test_one_expert_mxfp8_reduces_to_dense_swiglu_mlp():
    cfg = synth.custom_config(T=3, H=64, I=32, E=1, K=1, shared=0)
    W = _make_weights_mxfp8(cfg)
    x, l, _ = _inputs(cfg)
    res = moe.forward(x, l, None, W, cfg.I, cfg.E, cfg.K, 0, wfmt=moe.W_MXFP8)
    w13, w13s, w2, w2s = W(0)
    assert w13.shape == (2 * cfg.I, cfg.H) and w2.shape == (cfg.H, cfg.I)
    A = _decode_e4m3_by_torch(w13, w13s)   # [2I][H]
    B = _decode_e4m3_by_torch(w2, w2s)     # [H][I]
    xv = mxfp4.bf16_to_f64(x)
    for t in range(cfg.T):
        h = []
        for i in range(cfg.I):
            g = sum(A[i][k] * xv[t, k] for k in range(cfg.H))
            u = sum(A[cfg.I + i][k] * xv[t, k] for k in range(cfg.H))
            h.append(float(mxfp4.round_bf16(g / (1 + math.exp(-g)) * u)))
        for j in range(cfg.H):
            y = sum(B[j][i] * h[i] for i in range(cfg.I))
            assert abs(res["out_f64"][t, j] - y) <= 1e-12 * max(1.0, abs(y))


def test_mxfp8_layer_closer_to_unquantised_weights_than_mxfp4():
    """Both formats quantise the same fp32 draw; E4M3's 3 mantissa bits must
    land much nearer the unquantised-weight layer than E2M1's 1 bit."""
    cfg = synth.custom_config(T=12, H=128, I=64, E=6, K=2, shared=1)
    x, l, g = _inputs(cfg)
    raw = lambda e: (synth.expert_w13(cfg, e).double().numpy(), synth.expert_w2(cfg, e).double().numpy())
    ids, w = moe.route(l, g, cfg.K, 1)
    xv = mxfp4.bf16_to_f64(x)
    ref = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        for k in range(cfg.K + 1):
            w13, w2 = raw(int(ids[t, k]))
            acc = w13 @ xv[t]
            hh = acc[:cfg.I] / (1 + np.exp(-acc[:cfg.I])) * acc[cfg.I:]
            ref[t] += float(w[t, k]) * (w2 @ hh)
    o4 = moe.forward(x, l, g, _make_weights(cfg), cfg.I, cfg.E, cfg.K, 1)["out_f64"]
    o8 = moe.forward(x, l, g, _make_weights_mxfp8(cfg), cfg.I, cfg.E, cfg.K, 1, wfmt=moe.W_MXFP8)["out_f64"]
    e4 = np.linalg.norm(o4 - ref) / np.linalg.norm(ref)
    e8 = np.linalg.norm(o8 - ref) / np.linalg.norm(ref)
    assert e8 < 0.08 and e4 > 2.5 * e8, (e4, e8)


def test_shared_expert_fusion_equals_separate_dense_mlp():
    cfg = synth.custom_config(T=24, H=128, I=64, E=8, K=3, shared=1)
    W = _make_weights(cfg)
    x, l, g = _inputs(cfg)
    sig = (1 / (1 + np.exp(-g.astype(np.float64)))).astype(np.float32).astype(np.float64)
    dense = moe.expert_mlp(mxfp4.bf16_to_f64(x), *W(cfg.E), cfg.I, moe.ACT_BF16)
    for round_y in (False, True):
        fused = moe.forward(x, l, g, W, cfg.I, cfg.E, cfg.K, 1, round_y=round_y)
        routed = moe.forward(x, l, None, W, cfg.I, cfg.E, cfg.K, 0, round_y=round_y)
        d = mxfp4.round_bf16(dense) if round_y else dense
        want = routed["out_f64"] + sig[:, None] * d
        assert np.allclose(fused["out_f64"], want, rtol=1e-12, atol=1e-15)
        assert np.all(fused["ids"][:, cfg.K] == cfg.E)


def test_down_scale_linearity():
    cfg = synth.custom_config(T=16, H=128, I=64, E=8, K=2, shared=1)
    W = _make_weights(cfg)
    x, l, g = _inputs(cfg)
    base = moe.forward(x, l, g, W, cfg.I, cfg.E, cfg.K, 1)
    W2x = lambda e: (W(e)[0], W(e)[1], W(e)[2], (W(e)[3].astype(np.int32) + 1).astype(np.uint8))
    dbl = moe.forward(x, l, g, W2x, cfg.I, cfg.E, cfg.K, 1)
    assert np.array_equal(dbl["out_f64"], 2 * base["out_f64"])
    assert np.array_equal(mxfp4.bf16_to_f64(dbl["out"]), 2 * mxfp4.bf16_to_f64(base["out"]))


def test_token_permutation_and_expert_relabelling():
    cfg = synth.custom_config(T=20, H=128, I=64, E=8, K=3, shared=1)
    W = _make_weights(cfg)
    x, l, g = _inputs(cfg)
    base = moe.forward(x, l, g, W, cfg.I, cfg.E, cfg.K, 1)
    p = np.random.default_rng(4).permutation(cfg.T)
    perm = moe.forward(x[p], l[p], g[p], W, cfg.I, cfg.E, cfg.K, 1)
    assert np.array_equal(perm["out"], base["out"][p])
    q = np.random.default_rng(5).permutation(cfg.E)       # new expert j is old expert q[j]
    Wq = lambda e: W(int(q[e])) if e < cfg.E else W(e)
    rel = moe.forward(x, l[:, q], g, Wq, cfg.I, cfg.E, cfg.K, 1)
    assert np.array_equal(rel["out"], base["out"])
    assert np.array_equal(q[rel["ids"][:, :cfg.K]], base["ids"][:, :cfg.K])


def test_token_subset_matches_full():
    cfg = synth.custom_config(T=30, H=128, I=64, E=8, K=3, shared=1)
    W = _make_weights(cfg)
    x, l, g = _inputs(cfg)
    full = moe.forward(x, l, g, W, cfg.I, cfg.E, cfg.K, 1)
    sub = moe.forward(x, l, g, W, cfg.I, cfg.E, cfg.K, 1, tokens=[3, 17, 29])
    assert np.array_equal(sub["out"], full["out"][[3, 17, 29]])


def test_w4a4_close_to_w4a16():
    cfg = synth.custom_config(T=16, H=256, I=128, E=8, K=2, shared=1)
    W = _make_weights(cfg)
    x, l, g = _inputs(cfg)
    a16 = moe.forward(x, l, g, W, cfg.I, cfg.E, cfg.K, 1, act_fmt=moe.ACT_BF16)
    a4 = moe.forward(x, l, g, W, cfg.I, cfg.E, cfg.K, 1, act_fmt=moe.ACT_MXFP4)
    rel = np.linalg.norm(a4["out_f64"] - a16["out_f64"]) / np.linalg.norm(a16["out_f64"])
    assert 0.01 < rel < 0.25          # MXFP4 activations cost a few percent, not more


# ---------------------------------------------------------------- router GEMM

def _bits(a):
    return torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_router_logits_worked():
    # hand-worked: x = [[1, 2], [0.5, -1]], W rows [1, 0], [3, 0.25], [-2, 4]
    got = moe.router_logits(_bits([[1.0, 2.0], [0.5, -1.0]]), _bits([[1.0, 0.0], [3.0, 0.25], [-2.0, 4.0]]))
    assert np.array_equal(got, np.array([[1.0, 3.5, 6.0], [0.5, 1.25, -5.0]]))


def test_router_logits_unit_rows_pick_columns():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((7, 32)).astype(np.float32)
    wb = _bits(w)
    for i in (0, 5, 31):
        e = np.zeros((1, 32), dtype=np.float32)
        e[0, i] = 1.0
        got = moe.router_logits(_bits(e), wb)[0]
        want = torch.tensor(w[:, i]).to(torch.bfloat16).float().numpy().astype(np.float64)
        assert np.array_equal(got, want)


def test_router_logits_triple_loop():
    # plain loops over bf16 values; small integers times powers of two keep
    # every partial sum exact, so the two must agree bit for bit
    rng = np.random.default_rng(4)
    x = rng.integers(-8, 9, size=(3, 40)) * 0.25
    w = rng.integers(-8, 9, size=(5, 40)) * 0.125
    got = moe.router_logits(_bits(x), _bits(w))
    for t in range(3):
        for e in range(5):
            acc = 0.0
            for h in range(40):
                acc += float(x[t, h]) * float(w[e, h])
            assert got[t, e] == acc


def test_forward_from_h_continues_forward():
    """The layer from h onward, fed the oracle's own h, is the forward bit for
    bit (W4A16 and W4A4, y kept or rounded)."""
    for act in (moe.ACT_BF16, moe.ACT_MXFP4):
        cfg = synth.custom_config(T=20, H=128, I=64, E=8, K=3, shared=1, act_fmt=act,
                                  outlier_p=0.02 if act else 0.0)
        W = _make_weights(cfg)
        x, l, g = _inputs(cfg)
        for round_y in (False, True):
            full = moe.forward(x, l, g, W, cfg.I, cfg.E, cfg.K, 1, act_fmt=act, return_h=True,
                               round_y=round_y)
            rest = moe.forward_from_h(full["h"], l, g, W, cfg.I, cfg.E, cfg.K, 1, act_fmt=act,
                                      round_y=round_y)
            assert np.array_equal(rest["out_f64"], full["out_f64"])
            assert np.array_equal(rest["out"], full["out"])
