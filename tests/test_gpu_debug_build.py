"""The bound-checking debug build (libmoe_mxfp4_debug.so, compiled with
MOE_DEBUG; include/moe_mxfp4.h, moe_debug_flags) on the GPU.

- On every forward path (32-, 64-row GEMMs, W4A4 on both, MXFP8, routed
  from x, the full decode shape) and every per-step tile size its checks stay
  silent and its outputs equal the release build's bit for bit.
- An inverse map holding slot rows at or past T*Kp makes the combine set
  MOE_DEBUG_COMBINE and leave those slots out (as slots of weight 0 would be)
  instead of reading past the staged y.  The batch is sized so that even an
  unchecked read of those rows would stay inside the staged y's allocation."""
import sys

import pytest
import torch

import synth
from tests.helpers import DEV, Problem
from tests.test_gpu_canary import CASES, _stages, plain

pytestmark = pytest.mark.gpu


def ops():
    from mxfp4_routed_expert_top_amd import ops as o
    return o


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _forward(prob):
    o = ops()
    c = prob.cfg
    ids = torch.empty(c.T, c.Kp, dtype=torch.int32, device=DEV)
    w = torch.empty(c.T, c.Kp, dtype=torch.float32, device=DEV)
    out = prob.forward(topk_ids=ids, topk_weights=w)
    return [out, ids, w]


def _in_debug_build(fn):
    """fn() run against the debug build; returns (its result, the flags)."""
    o = ops()
    with o.using_library():
        torch.cuda.synchronize()
        assert o.debug_flags(reset=True) == 0, "flags left set by an earlier call"
        res = fn()
        torch.cuda.synchronize()
        flags = o.debug_flags(reset=True)
    return res, flags


@pytest.mark.parametrize("name", list(CASES) + ["decode"])
def test_debug_build_forward_silent_and_equal(name):
    prob = Problem(synth.CONFIGS["decode"] if name == "decode" else CASES[name])
    _say("debug build forward", name)
    want = _forward(prob)
    got, flags = _in_debug_build(lambda: _forward(prob))
    assert flags == 0, f"bound checks fired: {flags:#x}"
    for a, b in zip(got, want):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name,tm", [
    ("ragged", 32), ("tiled", 64), ("tiled", 128),
    ("w4a4", 32), ("w4a4_tiled", 64), ("w4a4_tiled", 128), ("w4a4_tiled", 256),
])
def test_debug_build_stages_silent_and_equal(name, tm):
    o = ops()
    prob = Problem(CASES[name])
    _say("debug build stages", name, "tile_m", tm)
    want = _stages(o, prob, tm, plain)
    got, flags = _in_debug_build(lambda: _stages(o, prob, tm, plain))
    assert flags == 0, f"bound checks fired: {flags:#x}"
    assert len(got) == len(want)
    for a, b in zip(got, want):
        assert torch.equal(a, b)


def test_debug_build_mxfp8_and_router_silent():
    o = ops()
    c = synth.custom_config("debug_mxfp8", T=200, H=512, I=256, E=8, K=3, shared=1)
    x = synth.activations(c).to(DEV)
    logits = synth.router_logits(c).to(DEV)
    gate = synth.gate_logits(c).to(DEV)
    u8 = dict(dtype=torch.uint8, device=DEV)
    w13 = torch.empty(c.Ep, 2 * c.I, c.H, **u8)
    w13s = torch.empty(c.Ep, 2 * c.I, c.H // 32, **u8)
    w2 = torch.empty(c.Ep, c.H, c.I, **u8)
    w2s = torch.empty(c.Ep, c.H, c.I // 32, **u8)
    for e in range(c.Ep):
        o.quantize_weights(synth.expert_w13(c, e, DEV), w13[e], w13s[e], o.W_MXFP8)
        o.quantize_weights(synth.expert_w2(c, e, DEV), w2[e], w2s[e], o.W_MXFP8)
    prob = Problem(c)
    wr = synth.router_weight(c).to(DEV)

    def run():
        a = o.mxfp8_forward(x, logits, gate, w13, w13s, w2, w2s, c.I, c.E, c.K, c.shared)
        b = o.mxfp4_forward_router(x, wr, prob.w13, prob.w13s, prob.w2, prob.w2s, c.I, c.E, c.K,
                                   c.shared, c.act_fmt)
        return [a, b]

    want = run()
    got, flags = _in_debug_build(run)
    assert flags == 0, f"bound checks fired: {flags:#x}"
    for a, b in zip(got, want):
        assert torch.equal(a, b)


def test_debug_build_combine_reports_rows_past_A():
    o = ops()
    c = synth.custom_config("debug_combine", T=128, H=256, I=128, E=16, K=8, shared=1)
    prob = Problem(c)
    T, H, Kp = c.T, c.H, c.Kp
    A = T * Kp
    # rows A + 3 and A + 15 of the staged y lie inside its allocation (fp16 part A*H*2
    # bytes, exponents A*H/32 after it: 15*H*2 < A*H/32 once A > 960)
    assert 15 * H * 2 < A * H // 32
    r = prob.stages()
    y, w, inv = r["y"], r["w"], r["align"]["inv"]
    bad = inv.clone()
    bad[0] = A + 3              # token 0, slot 0
    bad[5 * Kp + 2] = A + 15    # token 5, slot 2
    w0, fixed = w.clone(), inv.clone()
    w0[0, 0] = 0.0
    w0[5, 2] = 0.0
    want = o.combine(y, w0, fixed, T, H, Kp)           # those slots with weight 0, release build
    got, flags = _in_debug_build(lambda: o.combine(y, w, bad, T, H, Kp))
    assert flags & 4, f"the combine's check did not fire: {flags:#x}"
    assert not flags & ~4 & 0x7FFFFFFF
    g, wv = got.float(), want.float()
    assert torch.equal(g == wv, torch.ones_like(g, dtype=torch.bool))
