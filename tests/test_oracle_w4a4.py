"""Pins of the oracle's W4A4 composition: x quantised to MXFP4 and decoded,
the gate/up GEMM, SwiGLU rounded to bf16, h quantised to MXFP4 and decoded,
the down GEMM (OpenRelay "Gemma 4 31B on MI355X" post, sections
"Optimisation 3" and "Optimisation 4": activation + MXFP4 quantisation fused).

1. A hand-worked layer (tests/golden/w4a4_worked.json) whose output changes
   under each plausible mistake: dropping the x quantisation, quantising h
   before its bf16 rounding, one scale per row instead of per 32 elements,
   or skipping the h quantisation (each worked out in the file).
2. A one-expert layer on random data reduced to plain loops, with the MXFP4
   quantiser and the bf16 rounding written here a second way (log2 for the
   scale, midpoint thresholds for the codes, Python's exact round-half-even
   for bf16)."""
import json
import math
import os

import numpy as np

import synth
from oracle import moe, mxfp4

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "w4a4_worked.json")))
SH = GOLD["shape"]
H, I = SH["H"], SH["I"]


def golden_weights():
    """The hand-packed weight arrays (row-major MXFP4) of the worked layer."""
    w13 = np.zeros((2 * I, H // 2), np.uint8)
    w13s = np.zeros((2 * I, H // 32), np.uint8)
    w2 = np.zeros((H, I // 2), np.uint8)
    w2s = np.zeros((H, I // 32), np.uint8)
    for codes, scales, rows in ((w13, w13s, GOLD["w13_rows"]), (w2, w2s, GOLD["w2_rows"])):
        for r, spec in rows.items():
            if r == "note":
                continue
            scales[int(r)] = spec["scales"]
            for b, v in spec["bytes"].items():
                codes[int(r), int(b)] = v
    return w13, w13s, w2, w2s


def golden_dense():
    """The worked layer's weights as plain values (what the packed bytes mean)."""
    A = np.zeros((2 * I, H))
    B = np.zeros((H, I))
    for r, spec in GOLD["w13_rows"].items():
        if r != "note":
            A[int(r), spec["k"]] = spec["value"]
    for r, spec in GOLD["w2_rows"].items():
        if r != "note":
            for i, v in spec["nonzero"]:
                B[int(r), i] = v
    return A, B


def golden_x_bits():
    x = np.zeros((1, H), np.float32)
    for k, v in GOLD["x_nonzero"]:
        x[0, k] = v
    return (x.view(np.uint32) >> 16).astype(np.uint16)     # every value is bf16-exact


def sparse(pairs, n):
    v = np.zeros(n)
    for k, val in pairs:
        v[k] = val
    return v


def test_worked_weights_decode_to_their_values():
    w13, w13s, w2, w2s = golden_weights()
    A, B = golden_dense()
    assert np.array_equal(mxfp4.decode(w13, w13s), A)
    assert np.array_equal(mxfp4.decode(w2, w2s), B)
    # and the oracle's quantiser packs those values into the same bytes
    for (p, s), (wp, ws) in ((mxfp4.quantize(A), (w13, w13s)), (mxfp4.quantize(B), (w2, w2s))):
        assert np.array_equal(p, wp) and np.array_equal(s, ws)


def test_worked_x_quantisation():
    xq, xs = moe.quantize_activations(golden_x_bits())
    want_q = np.zeros(H // 2, np.uint8)
    for b, v in GOLD["xq_bytes"].items():
        want_q[int(b)] = v
    assert np.array_equal(xq[0], want_q)
    assert list(xs[0]) == GOLD["xs"]
    assert np.array_equal(mxfp4.decode(xq, xs)[0], sparse(GOLD["xq_values_nonzero"], H))


def test_worked_h_and_its_quantisation():
    w13, w13s, w2, w2s = golden_weights()
    a = mxfp4.decode(*moe.quantize_activations(golden_x_bits()))
    y, h = moe.expert_mlp(a, w13, w13s, w2, w2s, I, moe.ACT_MXFP4, return_h=True)
    assert np.array_equal(h[0], sparse(GOLD["h_nonzero"], I))
    hq, hs = mxfp4.quantize(h)
    want_q = np.zeros(I // 2, np.uint8)
    for b, v in GOLD["hq_bytes"].items():
        want_q[int(b)] = v
    assert np.array_equal(hq[0], want_q) and list(hs[0]) == GOLD["hs"]
    assert np.array_equal(mxfp4.decode(hq, hs)[0], sparse(GOLD["hq_values_nonzero"], I))
    assert np.array_equal(y[0], sparse(GOLD["out_nonzero"], H))


def test_worked_layer_output_bit_exact():
    w13, w13s, w2, w2s = golden_weights()
    res = moe.forward(golden_x_bits(), np.zeros((1, 1), np.float32), None,
                      lambda e: (w13, w13s, w2, w2s), I, 1, 1, 0, act_fmt=moe.ACT_MXFP4)
    want = sparse(GOLD["out_nonzero"], H)
    assert np.array_equal(mxfp4.bf16_to_f64(res["out"][0]), want)
    assert np.array_equal(res["out_f64"][0], want)
    assert res["w"][0, 0] == 1.0
    # each worked mistake would have changed the output
    for name, m in GOLD["mistakes"].items():
        if name == "note":
            continue
        diffs = [k for k in m if k.startswith("out") and m[k] != want[int(k[3:])]]
        assert diffs, name
    # the same layer as W4A16 (neither x nor h quantised) differs as well
    a16 = moe.forward(golden_x_bits(), np.zeros((1, 1), np.float32), None,
                      lambda e: (w13, w13s, w2, w2s), I, 1, 1, 0, act_fmt=moe.ACT_BF16)
    assert not np.array_equal(a16["out"], res["out"])


# --------------------------------------------- random data, plain loops --

MIDPOINTS = [(0.25, True, 0), (0.75, False, 1), (1.25, True, 2), (1.75, False, 3),
             (2.5, True, 4), (3.5, False, 5), (5.0, True, 6)]
VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def loop_quant_dequant(block):
    """MXFP4 quantise-then-decode of 32 values, written a second way: the
    scale exponent from log2, each magnitude's code from the midpoints
    between E2M1 values (a midpoint goes to the even code)."""
    amax = max(abs(v) for v in block)
    X = -127 if amax == 0 else max(-127, min(127, math.floor(math.log2(amax)) - 2))
    out = []
    for v in block:
        m = abs(v) / 2.0 ** X
        code = 7
        for bound, incl, c in reversed(MIDPOINTS):
            if (m <= bound) if incl else (m < bound):
                code = c
        out.append(math.copysign(VALUES[code] * 2.0 ** X, v))
    return out


def loop_bf16(v):
    """Nearest bf16 value of v (normal range), ties to even: 8 significant
    bits via Python's exact round-half-even on the scaled mantissa."""
    if v == 0:
        return v
    m, e = math.frexp(v)                 # v = m * 2^e, 0.5 <= |m| < 1
    return math.ldexp(round(m * 256), e - 8)


def test_one_expert_w4a4_reduces_to_plain_loops():
    cfg = synth.custom_config(T=3, H=64, I=64, E=1, K=1, shared=0, act_fmt=synth.ACT_MXFP4,
                              outlier_p=0.05)
    w13p = mxfp4.quantize(synth.expert_w13(cfg, 0).double().numpy())
    w2p = mxfp4.quantize(synth.expert_w2(cfg, 0).double().numpy())
    A = mxfp4.decode(*w13p).tolist()       # decode is pinned by the format tests
    B = mxfp4.decode(*w2p).tolist()
    x = synth.activations(cfg).view(__import__("torch").int16).numpy().view(np.uint16)
    l = synth.router_logits(cfg).numpy()
    res = moe.forward(x, l, None, lambda e: (*w13p, *w2p), cfg.I, 1, 1, 0,
                      act_fmt=moe.ACT_MXFP4)
    xv = mxfp4.bf16_to_f64(x)
    for t in range(cfg.T):
        a = []
        for b in range(0, cfg.H, 32):
            a += loop_quant_dequant(list(xv[t, b:b + 32]))
        h = []
        for i in range(cfg.I):
            g = sum(A[i][k] * a[k] for k in range(cfg.H))
            u = sum(A[cfg.I + i][k] * a[k] for k in range(cfg.H))
            h.append(loop_bf16(g / (1 + math.exp(-g)) * u))
        hin = []
        for b in range(0, cfg.I, 32):
            hin += loop_quant_dequant(h[b:b + 32])
        for j in range(cfg.H):
            y = sum(B[j][i] * hin[i] for i in range(cfg.I))       # top-1, weight 1: out = y
            assert abs(res["out_f64"][t, j] - y) <= 1e-12 * max(1.0, abs(y)), (t, j)
