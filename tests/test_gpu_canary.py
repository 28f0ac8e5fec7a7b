"""Canary-padded buffers: every output and workspace a call is given sits
between two 4 KiB guard bands of a known byte.  After the call each guard
must be unchanged (nothing written outside its buffer) and each output must
equal, bit for bit, what the same sequence of calls writes into plain
buffers (nothing read from outside the inputs, nothing left unwritten that
the result depends on).  Covers the one-call forwards (32-row, 64-row and
128-row GEMM paths, W4A4 on both, MXFP8, routed from x), every per-step
entry point at every tile size the kernels offer, the one-call routing +
grouping, and the step after the layer (partials summed, residual added,
RMSNorm)."""
import sys

import numpy as np
import pytest
import torch

import synth
from tests.helpers import DEV, Problem

pytestmark = pytest.mark.gpu

GUARD = 4096
CANARY = 0xA5


def ops():
    from mxfp4_routed_expert_top_amd import ops as o
    return o


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Guarded:
    """Allocator of guarded buffers (canary bytes before and after each)."""

    def __init__(self):
        self.bufs = []

    def __call__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        base = torch.full((n + 2 * GUARD,), CANARY, dtype=torch.uint8, device=DEV)
        self.bufs.append((base, n))
        return base[GUARD:GUARD + n].view(dtype).view(shape)

    def check(self):
        torch.cuda.synchronize()
        for i, (base, n) in enumerate(self.bufs):
            b = base.cpu().numpy()
            assert (b[:GUARD] == CANARY).all(), f"buffer {i}: written before its start"
            assert (b[GUARD + n:] == CANARY).all(), f"buffer {i}: written past its end"


def plain(shape, dtype):
    return torch.empty(shape, dtype=dtype, device=DEV)


CASES = {
    "ragged": synth.custom_config("canary_ragged", T=50, H=512, I=256, E=64, K=4, shared=1),
    "tiled": synth.custom_config("canary_tiled", T=300, H=512, I=256, E=8, K=3, shared=1),
    "w4a4": synth.custom_config("canary_w4a4", T=40, H=256, I=128, E=16, K=3, shared=1,
                                act_fmt=synth.ACT_MXFP4, outlier_p=0.01),
    "w4a4_tiled": synth.custom_config("canary_w4a4_tiled", T=300, H=512, I=256, E=8, K=3,
                                      shared=1, act_fmt=synth.ACT_MXFP4, outlier_p=0.002),
    "single_token": synth.custom_config("canary_one", T=1, H=384, I=256, E=64, K=6, shared=1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_forward_guards(name):
    """moe_mxfp4_forward: out, ids, weights and the workspace guarded."""
    o = ops()
    prob = Problem(CASES[name])
    c = prob.cfg
    _say("canary forward", name, "tile_m", o.gemm_tile_m(c.T, c.Kp, c.Ep, c.H, c.I, c.act_fmt))

    def run(alloc):
        out = alloc((c.T, c.H), torch.bfloat16)
        ids = alloc((c.T, c.Kp), torch.int32)
        w = alloc((c.T, c.Kp), torch.float32)
        ws = alloc((o.workspace_size(c.T, c.H, c.I, c.E, c.K, c.shared, c.act_fmt),), torch.uint8)
        prob.forward(out=out, topk_ids=ids, topk_weights=w, workspace=ws)
        return out, ids, w

    g = Guarded()
    got = run(g)
    g.check()
    want = run(plain)
    torch.cuda.synchronize()
    for a, b in zip(got, want):
        assert torch.equal(a, b)


def _stages(o, prob, tm, alloc):
    """Route, group (tile_m = tm), [quantise x], gate/up [with h quantised],
    down and combine through the per-step entry points, every buffer from
    alloc; returns the outputs."""
    c = prob.cfg
    T, H, I, Ep, Kp = c.T, c.H, c.I, c.Ep, c.Kp
    A = T * Kp
    r16 = (A + 15) // 16 * 16
    ids = alloc((T, Kp), torch.int32)
    w = alloc((T, Kp), torch.float32)
    o.route_topk(prob.logits, prob.gate, c.K, c.shared, topk_ids=ids, topk_weights=w)
    i32 = torch.int32
    al = dict(counts=alloc((Ep,), i32), offsets=alloc((Ep + 1,), i32), sorted=alloc((A,), i32),
              inv=alloc((A,), i32), tiles=alloc(((A + tm - 1) // tm + Ep, 2), i32),
              num_tiles=alloc((1,), i32),
              workspace=alloc((max(o.align_workspace_size(T, Kp, Ep), 1),), torch.uint8))
    o.align_sort(ids, Ep, tile_m=tm, out=al)
    u8 = torch.uint8
    res = [ids, w, al["counts"], al["offsets"], al["sorted"], al["inv"], al["num_tiles"]]
    if c.act_fmt == synth.ACT_BF16:
        h = alloc((A, I), torch.bfloat16)
        o.expert_gate_up(prob.x, None, o.ACT_BF16, al, prob.w13, prob.w13s, T, H, I, Ep, Kp, h=h)
        hin, hsc, act = h, None, o.ACT_BF16
        res.append(h)
    elif tm == 32:
        xq, xs = alloc((T, H // 2), u8), alloc((T, H // 32), u8)
        o.mxfp4_quantize(prob.x, xq, xs)
        h = alloc((A, I), torch.bfloat16)
        o.expert_gate_up(xq, xs, o.ACT_MXFP4, al, prob.w13, prob.w13s, T, H, I, Ep, Kp, h=h)
        hq, hs = alloc((A, I // 2), u8), alloc((A, I // 32), u8)
        o.mxfp4_quantize(h, hq, hs)
        hin, hsc, act = hq, hs, o.ACT_MXFP4
        res += [xq, xs, h, hq, hs]
    else:
        # (the blocked arrays' rows from A on are padding no call writes: zeroed
        # in both runs so that the arrays compare whole)
        xq, xs = alloc((r16, H // 2), u8).zero_(), alloc((r16, H // 32), u8).zero_()
        o.mxfp4_quantize_blocked(prob.x, al["inv"], Kp, A, xq, xs)
        hq, hs = alloc((r16, I // 2), u8).zero_(), alloc((r16, I // 32), u8).zero_()
        o.expert_gate_up_quant(xq, xs, al, prob.w13, prob.w13s, T, H, I, Ep, Kp, h_packed=hq,
                               h_scale=hs)
        hin, hsc, act = hq, hs, o.ACT_MXFP4_BLOCKED
        res += [xq, xs, hq, hs]
    y = alloc((o.staged_y_bytes(A, H),), u8)
    o.expert_down(hin, hsc, act, al, prob.w2, prob.w2s, T, H, I, Ep, Kp, y=y)
    out = alloc((T, H), torch.bfloat16)
    o.combine(y, w, al["inv"], T, H, Kp, out=out)
    return res + [y, out]


@pytest.mark.parametrize("name,tm", [
    ("ragged", 32), ("tiled", 64), ("tiled", 128),                 # bf16: 32-row, 64-row, 8-wave 128-row
    ("w4a4", 32), ("w4a4_tiled", 64), ("w4a4_tiled", 128), ("w4a4_tiled", 256),
])
def test_stage_guards(name, tm):
    """Every per-step entry point at tile size tm, all outputs guarded."""
    o = ops()
    prob = Problem(CASES[name])
    _say("canary stages", name, "tile_m", tm)
    g = Guarded()
    got = _stages(o, prob, tm, g)
    g.check()
    want = _stages(o, prob, tm, plain)
    torch.cuda.synchronize()
    assert len(got) == len(want)
    for a, b in zip(got, want):
        assert torch.equal(a, b)


@pytest.mark.parametrize("T,E,K,tm", [(1, 512, 10, 32), (4, 512, 14, 32), (16, 64, 3, 32),
                                      (16, 512, 10, 32),
                                      (30, 16, 3, 64), (64, 512, 10, 32), (300, 64, 4, 32)])
def test_route_align_guards(T, E, K, tm):
    """moe_route_align (a wave per token for the smallest batches, one 16-wave
    workgroup for the small ones, two launches beyond) with guarded outputs."""
    o = ops()
    gen = torch.Generator(device=DEV).manual_seed(T + E)
    logits = torch.randn(T, E, generator=gen, device=DEV)
    gate = torch.randn(T, generator=gen, device=DEV)
    Kp, Ep = K + 1, E + 1
    A = T * Kp
    _say("canary route_align", T, E, K, tm)

    def run(alloc):
        i32 = torch.int32
        ids, w = alloc((T, Kp), i32), alloc((T, Kp), torch.float32)
        al = dict(counts=alloc((Ep,), i32), offsets=alloc((Ep + 1,), i32), sorted=alloc((A,), i32),
                  inv=alloc((A,), i32), tiles=alloc(((A + tm - 1) // tm + Ep, 2), i32),
                  num_tiles=alloc((1,), i32),
                  workspace=alloc((max(o.align_workspace_size(T, Kp, Ep), 1),), torch.uint8))
        o.route_align(logits, gate, K, 1, tile_m=tm, topk_ids=ids, topk_weights=w, out=al)
        n = al["num_tiles"]
        return [ids, w, al["counts"], al["offsets"], al["sorted"], al["inv"], n, al["tiles"]]

    g = Guarded()
    got = run(g)
    g.check()
    want = run(plain)
    torch.cuda.synchronize()
    n = int(want[6].item())
    got[-1], want[-1] = got[-1][:n], want[-1][:n]       # (the table's rows past num_tiles are unused)
    for a, b in zip(got, want):
        assert torch.equal(a, b)


def test_layout_and_quantiser_guards():
    """moe_weights_to_native, the MXFP4 and MXFP8 quantisers (row-major and
    blocked with a row map) with guarded outputs."""
    o = ops()
    gen = torch.Generator(device=DEV).manual_seed(11)
    src = torch.randn(96, 384, generator=gen, device=DEV)
    codes = torch.randint(0, 256, (96, 192), dtype=torch.uint8, device=DEV)
    map_ = torch.randperm(96 * 2, device=DEV).to(torch.int32)

    def run(alloc):
        u8 = torch.uint8
        nat = alloc((96, 192), u8)
        o.weights_to_native(codes, out=nat)
        p4, s4 = alloc((96, 192), u8), alloc((96, 12), u8)
        o.mxfp4_quantize(src, p4, s4)
        p8, s8 = alloc((96, 384), u8), alloc((96, 12), u8)
        o.mxfp8_quantize(src, p8, s8)
        pb, sb = alloc((192, 192), u8), alloc((192, 12), u8)
        o.mxfp4_quantize_blocked(src.to(torch.bfloat16), map_, 2, 192, pb, sb)
        return nat, p4, s4, p8, s8, pb, sb

    g = Guarded()
    got = run(g)
    g.check()
    want = run(plain)
    torch.cuda.synchronize()
    for a, b in zip(got, want):
        assert torch.equal(a, b)


def test_mxfp8_and_router_forward_guards():
    """moe_mxfp8_forward and moe_mxfp4_forward_router (with its logits
    output and its own workspace) with guarded outputs."""
    o = ops()
    c = synth.custom_config("canary_mxfp8", T=200, H=512, I=256, E=8, K=3, shared=1)
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

    def run(alloc):
        out8 = alloc((c.T, c.H), torch.bfloat16)
        ws8 = alloc((o.mxfp8_workspace_size(c.T, c.H, c.I, c.E, c.K, c.shared),), torch.uint8)
        o.mxfp8_forward(x, logits, gate, w13, w13s, w2, w2s, c.I, c.E, c.K, c.shared, out=out8,
                        workspace=ws8)
        outr = alloc((c.T, c.H), torch.bfloat16)
        lg = alloc((c.T, c.Ep), torch.float32)
        wsr = alloc((o.workspace_size(c.T, c.H, c.I, c.E, c.K, c.shared, c.act_fmt),), torch.uint8)
        o.mxfp4_forward_router(x, wr, prob.w13, prob.w13s, prob.w2, prob.w2s, c.I, c.E, c.K,
                               c.shared, c.act_fmt, out=outr, logits_out=lg, workspace=wsr)
        return out8, outr, lg

    g = Guarded()
    got = run(g)
    g.check()
    want = run(plain)
    torch.cuda.synchronize()
    for a, b in zip(got, want):
        assert torch.equal(a, b)


@pytest.mark.parametrize("G,T,H", [(3, 37, 136), (8, 64, 4096), (2, 5, 16384)])
def test_residual_rmsnorm_guards(G, T, H):
    """moe_residual_rmsnorm: inputs, h and out in guarded buffers (in place
    and not), against the same calls on plain buffers."""
    o = ops()
    _say("canary residual_rmsnorm", G, T, H)
    p, r, g = synth.norm_inputs(G, T, H, seed=3 + G + H)

    def run(alloc, inplace):
        parts = []
        for i in range(G):
            t = alloc((T, H), torch.bfloat16)
            t.copy_(p[i])
            parts.append(t)
        res = alloc((T, H), torch.bfloat16)
        res.copy_(r)
        gam = alloc((H,), torch.bfloat16)
        gam.copy_(g)
        if inplace:
            out, _ = o.residual_rmsnorm(parts, gam, 1e-6, residual=res, residual_out=res,
                                        out=parts[0])
            return out, res
        hout = alloc((T, H), torch.bfloat16)
        out = alloc((T, H), torch.bfloat16)
        o.residual_rmsnorm(parts, gam, 1e-6, residual=res, residual_out=hout, out=out)
        return out, hout

    for inplace in (False, True):
        gd = Guarded()
        got = run(gd, inplace)
        gd.check()
        want = run(plain, inplace)
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a, b)
