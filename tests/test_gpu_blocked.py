"""MXFP4 activations in the blocked sorted-row order (include/moe_mxfp4.h,
moe_mxfp4_quantize_blocked, MOE_ACT_MXFP4_BLOCKED).

Bit-exact: the blocked quantiser against the oracle's quantiser put into the
blocked order by tests/helpers.blocked_order (with and without a row map;
rows nothing maps to keep their bytes), and the tiled GEMMs on blocked
activations against the same GEMMs on row-major ones (the same products in
the same order: only where the bytes come from differs), for every tile
size and reduction-length variant; and the gate/up GEMM with h quantised in
its epilogue against the blocked quantiser on its bf16 h."""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import mxfp4
from tests.helpers import DEV, Problem, bits, blocked_order, unblocked_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ops():
    from mxfp4_routed_expert_top_amd import ops as o
    return o


def _oracle_rows(v_f64):
    p, s = mxfp4.quantize(v_f64)
    return p, s


def _padded(a, rows):
    out = np.zeros((rows, a.shape[1]), dtype=a.dtype)
    out[:a.shape[0]] = a
    return out


@pytest.mark.parametrize("rows,cols,dtype", [(37, 384, torch.bfloat16), (16, 128, torch.float32),
                                             (300, 1536, torch.bfloat16)])
def test_quantize_blocked_rows(rows, cols, dtype):
    _say("quantize_blocked", rows, cols, dtype)
    g = torch.Generator().manual_seed(rows + cols)
    v = (torch.randn(rows, cols, generator=g) * 3).to(dtype)
    v[0, :32] = 0                                  # an all-zero block
    r16 = (rows + 15) // 16 * 16
    pk = torch.full((r16, cols // 2), 0xAB, dtype=torch.uint8, device=DEV)
    sc = torch.full((r16, cols // 32), 0xCD, dtype=torch.uint8, device=DEV)
    ops().mxfp4_quantize_blocked(v.to(DEV), packed=pk, scales=sc)
    torch.cuda.synchronize()
    wp, ws = _oracle_rows(v.double().numpy())
    # rows past `rows` keep their fill bytes
    fill_p = np.full((r16, cols // 2), 0xAB, np.uint8)
    fill_s = np.full((r16, cols // 32), 0xCD, np.uint8)
    fill_p[:rows], fill_s[:rows] = wp, ws
    ep, es = blocked_order(fill_p, fill_s)
    assert np.array_equal(pk.cpu().numpy(), ep)
    assert np.array_equal(sc.cpu().numpy(), es)


def test_quantize_blocked_row_map():
    """Each token into its sorted slots (the grouping's inverse map), and map
    values out of range writing nothing."""
    T, Kp, H, Ep = 50, 3, 256, 7
    g = torch.Generator().manual_seed(11)
    x = (torch.randn(T, H, generator=g) * 2).to(torch.bfloat16)
    ids = torch.randint(0, Ep, (T, Kp), generator=g, dtype=torch.int32)
    al = ops().align_sort(ids.to(DEV), Ep)
    inv = al["inv"]
    A = T * Kp
    r16 = (A + 15) // 16 * 16
    pk, sc = ops().mxfp4_quantize_blocked(x.to(DEV), inv, Kp, A)
    torch.cuda.synchronize()
    wp, ws = _oracle_rows(mxfp4.bf16_to_f64(bits(x)))
    invn = inv.cpu().numpy()
    rp = np.zeros((r16, H // 2), np.uint8)
    rs = np.zeros((r16, H // 32), np.uint8)
    for a in range(A):
        rp[invn[a]], rs[invn[a]] = wp[a // Kp], ws[a // Kp]
    # rows A .. r16 are padding nothing maps to: compare the written rows only
    gp, gs = unblocked_rows(pk.cpu().numpy(), sc.cpu().numpy())
    assert np.array_equal(gp[:A], rp[:A]) and np.array_equal(gs[:A], rs[:A])

    bad = inv.clone()
    bad[0] = -1                                    # token 0, slot 0: nowhere
    bad[1] = A + 5                                 # token 0, slot 1: past out_rows
    pk2 = torch.full_like(pk, 0x5A)
    sc2 = torch.full_like(sc, 0x5A)
    ops().mxfp4_quantize_blocked(x.to(DEV), bad, Kp, A, pk2, sc2)
    torch.cuda.synchronize()
    up, us = unblocked_rows(pk2.cpu().numpy(), sc2.cpu().numpy())
    for a in range(A):
        p = invn[a]
        if a in (0, 1):
            assert (up[p] == 0x5A).all() and (us[p] == 0x5A).all()
        else:
            assert np.array_equal(up[p], rp[p]) and np.array_equal(us[p], rs[p])
    assert (up[A:] == 0x5A).all() and (us[A:] == 0x5A).all()


@pytest.mark.parametrize("tile_m,T,H,I,E,K", [
    (64, 150, 512, 256, 8, 3),          # 64-row tiles
    (128, 300, 512, 256, 8, 3),         # 128-row tiles, reductions <= 2048
    (128, 200, 2560, 2560, 4, 1),       # reductions <= 6144 (gate/up and down)
    (128, 200, 6400, 6400, 4, 1),       # whole-K variant (reductions > 6144)
    (256, 300, 512, 256, 8, 3),         # 256-row tiles
])
def test_gemms_blocked_equal_row_major(tile_m, T, H, I, E, K):
    cfg = synth.custom_config(f"blk{tile_m}_{H}", T=T, H=H, I=I, E=E, K=K, shared=1,
                              act_fmt=synth.ACT_MXFP4, outlier_p=0.002)
    _say("blocked gemms tile_m", tile_m, "T", T, "H", H, "I", I)
    prob = Problem(cfg)
    c = prob.cfg
    o = ops()
    ids, w = o.route_topk(prob.logits, prob.gate, c.K, c.shared)
    al = o.align_sort(ids, c.Ep, tile_m=tile_m)
    A = c.T * c.Kp
    xq, xs = o.mxfp4_quantize(prob.x)
    h_row = o.expert_gate_up(xq, xs, o.ACT_MXFP4, al, prob.w13, prob.w13s, c.T, c.H, c.I, c.Ep,
                             c.Kp)
    xb, xbs = o.mxfp4_quantize_blocked(prob.x, al["inv"], c.Kp, A)
    h_blk = o.expert_gate_up(xb, xbs, o.ACT_MXFP4_BLOCKED, al, prob.w13, prob.w13s, c.T, c.H,
                             c.I, c.Ep, c.Kp)
    torch.cuda.synchronize()
    assert np.array_equal(bits(h_blk), bits(h_row))
    # h quantised in the gate/up epilogue == the blocked quantiser on the bf16 h
    fq, fs = o.expert_gate_up_quant(xb, xbs, al, prob.w13, prob.w13s, c.T, c.H, c.I, c.Ep, c.Kp)
    qq, qs = o.mxfp4_quantize_blocked(h_blk)
    torch.cuda.synchronize()
    pq, ps = o.expert_gate_up_quant(xq, xs, al, prob.w13, prob.w13s, c.T, c.H, c.I, c.Ep, c.Kp,
                                    act_fmt=o.ACT_MXFP4)     # per-token activation rows
    torch.cuda.synchronize()
    fq, fs = unblocked_rows(fq.cpu().numpy(), fs.cpu().numpy())
    pq, ps = unblocked_rows(pq.cpu().numpy(), ps.cpu().numpy())
    qq, qs = unblocked_rows(qq.cpu().numpy(), qs.cpu().numpy())
    assert np.array_equal(fq[:A], qq[:A]) and np.array_equal(fs[:A], qs[:A])
    assert np.array_equal(pq[:A], qq[:A]) and np.array_equal(ps[:A], qs[:A])
    hq, hs = o.mxfp4_quantize(h_row)
    y_row = o.expert_down(hq, hs, o.ACT_MXFP4, al, prob.w2, prob.w2s, c.T, c.H, c.I, c.Ep, c.Kp)
    hb, hbs = o.mxfp4_quantize_blocked(h_row)
    y_blk = o.expert_down(hb, hbs, o.ACT_MXFP4_BLOCKED, al, prob.w2, prob.w2s, c.T, c.H, c.I,
                          c.Ep, c.Kp)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y_blk), bits(y_row))
