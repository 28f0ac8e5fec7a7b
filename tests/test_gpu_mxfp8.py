"""MXFP8 expert weights (W8A16) through the C ABI against the CPU oracle.

Bit-exact: the MXFP8 packing (GPU quantiser vs the oracle's), routing ids
and the grouping tables.  Within tolerance, as for W4A16 (the arithmetic is
the same: exact dequantised weights times bf16 activations, fp32 sums, h
and y rounded to bf16): routing weights 1e-6, layer output relative L2 <=
5e-3 and max abs <= 2e-2 x RMS of the oracle output."""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import moe, mxfp4, mxfp8
from tests.helpers import (DEV, MAX_ABS_RMS, REL_L2, W_ATOL, bits, max_abs_over_rms, native_order,
                           oracle_pack, oracle_pack_all, rel_l2)

pytestmark = pytest.mark.gpu

TOL = REL_L2[synth.ACT_BF16]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ops():
    from mxfp4_routed_expert_top_amd import ops as o
    return o


class Problem8:
    """One workload with MXFP8 weights packed on the GPU, and lazily by the
    oracle's quantiser from the same draws."""

    def __init__(self, cfg, logits=None):
        c = self.cfg = cfg
        self.x_cpu = synth.activations(c)
        self.logits_cpu = synth.router_logits(c) if logits is None else logits
        self.gate_cpu = synth.gate_logits(c)
        self.x = self.x_cpu.to(DEV)
        self.logits = self.logits_cpu.to(DEV)
        self.gate = None if self.gate_cpu is None else self.gate_cpu.to(DEV)
        u8 = dict(dtype=torch.uint8, device=DEV)
        self.w13 = torch.empty(c.Ep, 2 * c.I, c.H, **u8)
        self.w13s = torch.empty(c.Ep, 2 * c.I, c.H // 32, **u8)
        self.w2 = torch.empty(c.Ep, c.H, c.I, **u8)
        self.w2s = torch.empty(c.Ep, c.H, c.I // 32, **u8)
        for e in range(c.Ep):
            ops().quantize_weights(synth.expert_w13(c, e, DEV), self.w13[e], self.w13s[e],
                                   ops().W_MXFP8)
            ops().quantize_weights(synth.expert_w2(c, e, DEV), self.w2[e], self.w2s[e],
                                   ops().W_MXFP8)
        torch.cuda.synchronize()

    def oracle_weights(self, e: int):
        return oracle_pack(self.cfg, e, synth.W_MXFP8)

    def oracle(self, tokens=None, return_h=False):
        c = self.cfg
        logits = self.logits_cpu.numpy()
        gate = None if self.gate_cpu is None else self.gate_cpu.numpy()
        ids, _ = moe.route(logits, gate, c.K, c.shared)
        oracle_pack_all(c, np.unique(ids if tokens is None else ids[np.asarray(tokens)]),
                        synth.W_MXFP8)
        return moe.forward(bits(self.x_cpu), logits, gate, self.oracle_weights, c.I, c.E, c.K,
                           c.shared, moe.ACT_BF16, tokens=tokens, wfmt=moe.W_MXFP8,
                           return_h=return_h)

    def forward(self, **kw):
        c = self.cfg
        return ops().mxfp8_forward(self.x, self.logits, self.gate, self.w13, self.w13s, self.w2,
                                   self.w2s, c.I, c.E, c.K, c.shared, **kw)

    def stages(self, **kw):
        c = self.cfg
        return ops().forward_stages(self.x, self.logits, self.gate, self.w13, self.w13s, self.w2,
                                    self.w2s, c.I, c.E, c.K, c.shared, ops().ACT_BF16,
                                    wfmt=ops().W_MXFP8, **kw)


# ------------------------------------------------------------- quantiser --

def _special_blocks():
    """Every midpoint between neighbouring E4M3 magnitudes (ties), values
    above 448 (saturation), signed zeros, subnormal-range values, at several
    block exponents; each block opens with 256 so that X = 0 before scaling."""
    g = mxfp8.GRID
    mids = list((g[:-1] + g[1:]) / 2) + [452.0, 464.0, 480.0, 496.0, 510.0, -0.0, 0.0,
                                         2.0 ** -10, 3 * 2.0 ** -10, -(2.0 ** -10)]
    rows = []
    for X in [-110, -100, -9, -1, 0, 5, 100]:          # all values stay normal in bf16
        for i in range(0, len(mids), 31):
            blk = np.zeros(32)
            blk[0] = 256.0
            part = np.array(mids[i:i + 31])
            blk[1:1 + part.size] = part * np.where(np.arange(part.size) % 2, -1, 1)
            rows.append(blk * 2.0 ** X)
    rows.append(np.zeros(32))
    rows.append(-np.zeros(32))
    if len(rows) % 2:
        rows.append(np.zeros(32))
    return np.array(rows).reshape(-1, 64)      # two blocks per row


@pytest.mark.parametrize("kind", ["weights_f32", "act_bf16", "special_f32", "special_bf16"])
def test_mxfp8_quantize_bit_exact(kind):
    _say("mxfp8 quantize", kind)
    g = torch.Generator().manual_seed(21)
    if kind == "weights_f32":
        v = torch.randn(512, 1024, generator=g) * 0.02
    elif kind == "act_bf16":
        v = torch.randn(300, 2048, generator=g)
        v = torch.where(torch.rand(300, 2048, generator=g) < 0.01, v * 50, v).to(torch.bfloat16)
    else:
        sb = _special_blocks()
        v = torch.from_numpy(sb.astype(np.float32))
        assert np.array_equal(v.double().numpy(), sb)           # exact in fp32
        if kind == "special_bf16":
            v = v.to(torch.bfloat16)
            assert np.array_equal(v.double().numpy(), sb)       # and in bf16
    q, s = ops().mxfp8_quantize(v.to(DEV))
    want_q, want_s = mxfp8.quantize(v.double().numpy())
    assert np.array_equal(s.cpu().numpy(), want_s)
    assert np.array_equal(q.cpu().numpy(), want_q)


# -------------------------------------------------------------- the layer --

SMALL = {
    "tiny": synth.CONFIGS["tiny"],
    "ragged": synth.custom_config("ragged8", T=50, H=512, I=256, E=64, K=4, shared=1),
    "no_shared_k1": synth.custom_config("no_shared_k1_8", T=33, H=256, I=128, E=8, K=1, shared=0),
    "one_expert": synth.custom_config("one_expert8", T=7, H=128, I=128, E=1, K=1, shared=0),
    "single_token": synth.custom_config("single_token8", T=1, H=384, I=256, E=64, K=6, shared=1),
    "sparse": synth.custom_config("sparse8", T=3, H=256, I=128, E=300, K=2, shared=1),
    # many 32-row tiles per expert, several 16-row subtiles per tile, odd K chunk count
    "big_groups": synth.custom_config("big_groups8", T=300, H=384, I=384, E=16, K=3, shared=1),
    # groups large enough for the LDS-tiled kernels (64- and 128-row tiles)
    "tiled64": synth.custom_config("tiled64_8", T=200, H=256, I=128, E=24, K=4, shared=1),
    "tiled128": synth.custom_config("tiled128_8", T=300, H=512, I=256, E=16, K=3, shared=1),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_mxfp8_layer_small(name):
    _say("mxfp8 layer", name)
    prob = Problem8(SMALL[name])
    c = prob.cfg
    for e in {0, c.Ep - 1}:                    # the two packings agree bit for bit
        w = prob.oracle_weights(e)
        assert np.array_equal(prob.w13[e].cpu().numpy(), native_order(w[0], 2))
        assert np.array_equal(prob.w13s[e].cpu().numpy(), w[1])
        assert np.array_equal(prob.w2[e].cpu().numpy(), native_order(w[2], 2))
        assert np.array_equal(prob.w2s[e].cpu().numpy(), w[3])
    r = prob.stages()
    out = prob.forward()
    torch.cuda.synchronize()
    want = prob.oracle()
    assert np.array_equal(bits(out), bits(r["out"]))          # one call == per-stage calls
    assert np.array_equal(r["ids"].cpu().numpy(), want["ids"])
    assert np.max(np.abs(r["w"].cpu().numpy() - want["w"])) <= W_ATOL
    assert np.array_equal(r["align"]["sorted"].cpu().numpy(), want["sorted"])
    e_rel = rel_l2(bits(out), want["out"])
    e_max = max_abs_over_rms(bits(out), want)
    _say(f"  {name}: rel_l2 {e_rel:.2e}  max_abs/rms {e_max:.2e}")
    assert e_rel <= TOL
    assert e_max <= MAX_ABS_RMS


def test_mxfp8_layer_empty_batch():
    cfg = synth.custom_config("empty8", T=1)
    prob = Problem8(cfg)
    x = torch.empty(0, cfg.H, dtype=torch.bfloat16, device=DEV)
    l = torch.empty(0, cfg.E, dtype=torch.float32, device=DEV)
    g = torch.empty(0, dtype=torch.float32, device=DEV)
    out = ops().mxfp8_forward(x, l, g, prob.w13, prob.w13s, prob.w2, prob.w2s, cfg.I, cfg.E,
                              cfg.K, cfg.shared)
    assert out.shape == (0, cfg.H)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode_mxfp8", "prefill_mxfp8"])
def test_mxfp8_layer_full_size(name):
    """The MXFP8 workloads (T = 64 on the weight-streaming kernels, T = 1536 on
    the 64-row LDS-tiled ones) in the launch configuration the bench times:
    routing and grouping bit-exact, h of every sorted row and every token's
    output against the oracle."""
    cfg = synth.CONFIGS[name]
    _say("mxfp8 full", name, cfg.T, "tile_m",
         ops().mxfp8_gemm_tile_m(cfg.T, cfg.Kp, cfg.Ep, cfg.H, cfg.I))
    prob = Problem8(cfg)
    ids = torch.empty(cfg.T, cfg.Kp, dtype=torch.int32, device=DEV)
    w = torch.empty(cfg.T, cfg.Kp, dtype=torch.float32, device=DEV)
    out = prob.forward(topk_ids=ids, topk_weights=w)
    r = prob.stages()
    torch.cuda.synchronize()
    assert torch.equal(out, r["out"])
    _say("  GPU done")
    want = prob.oracle(return_h=True)
    _say(f"  oracle done ({want['seconds']:.1f} s)")
    assert np.array_equal(ids.cpu().numpy(), want["ids"])
    assert np.max(np.abs(w.cpu().numpy() - want["w"])) <= W_ATOL
    assert np.array_equal(r["align"]["sorted"].cpu().numpy(), want["sorted"])
    hg, hw = bits(r["h"]), want["h"]
    h_rel = rel_l2(hg, hw)
    h_same = float(np.mean(hg == hw))
    _say(f"  h rel_l2 {h_rel:.2e}, bit-identical {h_same:.5f}")
    assert h_rel <= 2e-3 and h_same >= 0.99
    got = bits(out)
    e_rel = rel_l2(got, want["out"])
    e_max = max_abs_over_rms(got, want)
    _say(f"  {name}: all {cfg.T} tokens: rel_l2 {e_rel:.2e}  max_abs/rms {e_max:.2e}")
    assert e_rel <= TOL and e_max <= MAX_ABS_RMS
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("tile_m", [32, 64, 128])
def test_mxfp8_gemm_kernels_for_every_tile_size(tile_m):
    """The MXFP8 per-step entry points with each tile size against the oracle."""
    cfg = synth.custom_config("tiles8", T=150, H=512, I=256, E=8, K=3, shared=1)
    _say("mxfp8 tile_m", tile_m)
    prob = Problem8(cfg)
    c, o = prob.cfg, ops()
    ids, w = o.route_topk(prob.logits, prob.gate, c.K, c.shared)
    al = o.align_sort(ids, c.Ep, tile_m=tile_m)
    h = o.mxfp8_expert_gate_up(prob.x, al, prob.w13, prob.w13s, c.T, c.H, c.I, c.Ep, c.Kp)
    y = o.mxfp8_expert_down(h, al, prob.w2, prob.w2s, c.T, c.H, c.I, c.Ep, c.Kp)
    out = o.combine(y, w, al["inv"], c.T, c.H, c.Kp)
    torch.cuda.synchronize()
    want = prob.oracle()
    e_rel = rel_l2(bits(out), want["out"])
    e_max = max_abs_over_rms(bits(out), want)
    _say(f"  tile_m {tile_m}: rel_l2 {e_rel:.2e}  max_abs/rms {e_max:.2e}")
    assert e_rel <= TOL and e_max <= MAX_ABS_RMS
