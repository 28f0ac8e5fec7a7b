"""The router GEMM + routing call (moe_route_topk_gemm) against the oracle.

The GPU's logits are fp32 sums of exact bf16 products, so they are compared
with the oracle's exact fp64 logits within the fp32 summation bound
|fl(sum p) - sum p| <= gamma_H * sum |p| (gamma_n = n u / (1 - n u),
u = 2^-24, n = H terms).  The selection is an integer decision taken on
floating point, so both sides take it on the same fp32 logits: the oracle
routes the GPU's logits and ids must match bit for bit, weights within
1e-6.  The call must also agree exactly with moe_route_topk on those logits
and give the same bits when repeated."""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import moe
from tests.helpers import DEV, W_ATOL, bits

pytestmark = pytest.mark.gpu

CASES = {
    # name: (T, H, E, K, shared)
    "tiny": (8, 256, 16, 2, 0),
    "odd": (37, 384, 100, 7, 1),
    "single_token": (1, 128, 64, 6, 1),
    "decode": (64, 4096, 512, 10, 1),
    "prefill": (1536, 4096, 512, 10, 1),
    "w4a4_shape": (300, 6144, 256, 8, 1),
    "max_experts": (70, 512, 1024, 31, 1),
    # enough token tiles for the wide (unsplit) router kernel; ragged last tile
    "wide": (4200, 256, 300, 5, 1),
}


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", list(CASES))
def test_router_gemm_routing(name):
    from mxfp4_routed_expert_top_amd import ops
    T, H, E, K, shared = CASES[name]
    _say("router", name, "T", T, "H", H, "E", E, "K", K, "shared", shared)
    cfg = synth.custom_config(f"router_{name}", T=T, H=H, I=128, E=E, K=K, shared=shared)
    x = synth.activations(cfg)
    w = synth.router_weight(cfg)
    xd, wd = x.to(DEV), w.to(DEV)
    logits = torch.empty(T, E + shared, dtype=torch.float32, device=DEV)
    ids, wts, _ = ops.route_topk_gemm(xd, wd, K, shared, logits_out=logits)
    torch.cuda.synchronize()
    _say("  done on the GPU")
    lg = logits.cpu().numpy().astype(np.float64)
    exact = moe.router_logits(bits(x), bits(w))
    mag = np.abs(bits_to(x)) @ np.abs(bits_to(w)).T       # sum |p| per logit
    u = 2.0 ** -24
    gamma = H * u / (1 - H * u)
    err = np.abs(lg - exact)
    assert np.all(err <= gamma * mag + 1e-30), float(np.max(err / (gamma * mag + 1e-30)))
    _say(f"  logits: max |err| {err.max():.3e}, max err / bound {np.max(err / (gamma * mag + 1e-30)):.3f}")
    # the selection, on the same fp32 logits
    l32 = logits.cpu().numpy()
    want_ids, want_w = moe.route(l32[:, :E], l32[:, E] if shared else None, K, shared)
    assert np.array_equal(ids.cpu().numpy(), want_ids)
    assert np.max(np.abs(wts.cpu().numpy() - want_w)) <= W_ATOL
    # same as routing the returned logits directly
    gate = logits[:, E].contiguous() if shared else None
    ids2, w2 = ops.route_topk(logits[:, :E].contiguous(), gate, K, shared)
    assert torch.equal(ids, ids2) and torch.equal(wts, w2)
    # repeatable bit for bit
    logits_b = torch.empty_like(logits)
    ids3, w3, _ = ops.route_topk_gemm(xd, wd, K, shared, logits_out=logits_b)
    assert torch.equal(logits, logits_b) and torch.equal(ids, ids3) and torch.equal(wts, w3)


def bits_to(t: torch.Tensor) -> np.ndarray:
    return t.float().numpy().astype(np.float64)


def test_router_gemm_without_logits_out_and_empty_batch():
    from mxfp4_routed_expert_top_amd import ops
    cfg = synth.custom_config("router_nolog", T=20, H=256, I=128, E=32, K=4, shared=1)
    xd, wd = synth.activations(cfg).to(DEV), synth.router_weight(cfg).to(DEV)
    ids, wts, lo = ops.route_topk_gemm(xd, wd, 4, 1)
    logits = torch.empty(20, 33, dtype=torch.float32, device=DEV)
    ids2, wts2, _ = ops.route_topk_gemm(xd, wd, 4, 1, logits_out=logits)
    assert lo is None and torch.equal(ids, ids2) and torch.equal(wts, wts2)
    e = torch.empty(0, 256, dtype=torch.bfloat16, device=DEV)
    ids0, w0, _ = ops.route_topk_gemm(e, wd, 4, 1)
    assert ids0.shape == (0, 5) and w0.shape == (0, 5)


@pytest.mark.parametrize("name", ["tiny", "tiled128", "w4a4_small", "decode"])
def test_forward_router_equals_forward_on_its_logits(name):
    """The layer routed from x equals the layer fed the logits the router
    GEMM produced (bit for bit: the same kernels after routing), and matches
    the oracle's layer on those logits."""
    from mxfp4_routed_expert_top_amd import ops
    from tests.helpers import (MAX_ABS_RMS, REL_L2, Problem, max_abs_over_rms, oracle_pack_all,
                               rel_l2)
    cfg = {"tiny": synth.CONFIGS["tiny"],
           "tiled128": synth.custom_config("r_tiled128", T=300, H=512, I=256, E=16, K=3, shared=1),
           "w4a4_small": synth.custom_config("r_w4a4", T=40, H=256, I=128, E=16, K=3, shared=1,
                                             act_fmt=synth.ACT_MXFP4, outlier_p=0.01),
           "decode": synth.CONFIGS["decode"]}[name]
    _say("forward_router", name)
    prob = Problem(cfg)
    x = prob.x
    wr = synth.router_weight(cfg).to(DEV)
    wts = (prob.w13, prob.w13s, prob.w2, prob.w2s)
    logits = torch.empty(cfg.T, cfg.Ep, dtype=torch.float32, device=DEV)
    out_r = ops.mxfp4_forward_router(x, wr, *wts, cfg.I, cfg.E, cfg.K, cfg.shared, cfg.act_fmt,
                                     logits_out=logits)
    gate = logits[:, cfg.E].contiguous() if cfg.shared else None
    out_l = ops.mxfp4_forward(x, logits[:, :cfg.E].contiguous(), gate, *wts, cfg.I, cfg.E, cfg.K,
                              cfg.shared, cfg.act_fmt)
    torch.cuda.synchronize()
    assert torch.equal(out_r, out_l)
    l32 = logits.cpu().numpy()
    gate_np = l32[:, cfg.E] if cfg.shared else None
    _say("  GPU done; oracle on every token")
    ids_np, _ = moe.route(l32[:, :cfg.E], gate_np, cfg.K, cfg.shared)
    oracle_pack_all(cfg, np.unique(ids_np))
    want = moe.forward(bits(prob.x_cpu), l32[:, :cfg.E], gate_np, prob.oracle_weights, cfg.I,
                       cfg.E, cfg.K, cfg.shared, cfg.act_fmt)
    got = bits(out_r.cpu())
    e_rel, e_max = rel_l2(got, want["out"]), max_abs_over_rms(got, want)
    _say(f"  {name}: rel_l2 {e_rel:.2e}  max_abs/rms {e_max:.2e}")
    assert e_rel <= REL_L2[cfg.act_fmt] and e_max <= MAX_ABS_RMS
