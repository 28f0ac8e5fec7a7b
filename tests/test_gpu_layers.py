"""Several MoE layers in one call (moe_mxfp4_forward_layers) against the same
layers called one at a time, against the oracle, and under HIP graph capture.

Each layer routes from its input through its own router rows, so a layer's
top-K is an integer decision taken on floating-point logits.  As in the
router tests, the oracle takes that decision on the GPU's own fp32 logits
of the layer (and the GPU's output of the previous layer as the layer's
input); the multi-layer call must equal the chain of single-layer router
calls bit for bit, with and without the cache prefetch, and every graph
replay must equal the eager result.

Tolerance of a layer against the oracle: relative L2 as for one layer.
Layer 0 (fed the N(0,1) activations) keeps the layer's max-abs bound,
2e-2 x RMS of the oracle's output.  For later layers the max-abs bound is
taken per element against max(|want|, RMS(want)): both sides round y and
out to bf16 at the same points, so they differ by rare one-ulp rounding
flips, and a flip is proportional to the element it hits.  A layer fed by
another layer (no residual or norm in between) gives heavy-tailed outputs
(max/RMS 6-9 by the third layer, against ~4 for N(0,1) inputs), where one
flip at the largest element alone is 2.5-3.5% of the RMS."""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import moe, mxfp4
from tests.helpers import (DEV, MAX_ABS_RMS, REL_L2, W_ATOL, bf16_ulp, bits,
                           check_residual_rmsnorm, max_abs_over_rms, oracle_pack, oracle_pack_all,
                           rel_l2)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ops():
    from mxfp4_routed_expert_top_amd import ops as o
    return o


def max_abs_elementwise(got_bits, want) -> float:
    """max_j (|got_j - want_f64_j| - ulp(got_j) / 2) / max(|want_j|, RMS(want)):
    as the layer's max-abs measure (beyond the output's own rounding), taken
    per element against the element's own size."""
    g = mxfp4.bf16_to_f64(got_bits)
    w = mxfp4.bf16_to_f64(want["out"])
    f = np.asarray(want["out_f64"], dtype=np.float64)
    rms = float(np.sqrt(np.mean(w * w)))
    err = np.maximum(np.abs(g - f) - 0.5 * bf16_ulp(g), 0.0)
    return float(np.max(err / np.maximum(np.abs(w), max(rms, 1e-300))))


class Layers:
    """L layers of one workload's shapes, each with its own weights and
    router rows (synth.layer_config), packed on the GPU, plus the oracle's
    own packing of the same draws."""

    def __init__(self, cfg, L):
        self.cfg, self.L = cfg, L
        c = cfg
        self.x_cpu = synth.activations(c)
        self.x = self.x_cpu.to(DEV)
        self.w = []
        u8 = dict(dtype=torch.uint8, device=DEV)
        for l in range(L):
            lc = synth.layer_config(c, l)
            w13 = torch.empty(c.Ep, 2 * c.I, c.H // 2, **u8)
            w13s = torch.empty(c.Ep, 2 * c.I, c.H // 32, **u8)
            w2 = torch.empty(c.Ep, c.H, c.I // 2, **u8)
            w2s = torch.empty(c.Ep, c.H, c.I // 32, **u8)
            for e in range(c.Ep):
                ops().quantize_weights(synth.expert_w13(lc, e, DEV), w13[e], w13s[e])
                ops().quantize_weights(synth.expert_w2(lc, e, DEV), w2[e], w2s[e])
            self.w.append((synth.router_weight(lc).to(DEV), w13, w13s, w2, w2s))
        torch.cuda.synchronize()

    def oracle_weights(self, l, e):
        return oracle_pack(synth.layer_config(self.cfg, l), e)

    def multi(self, prefetch, **kw):
        c = self.cfg
        return ops().mxfp4_forward_layers(self.x, self.w, c.I, c.E, c.K, c.shared, c.act_fmt,
                                          prefetch=prefetch, **kw)

    def chain(self):
        """The layers one call at a time: (input, logits, output) per layer."""
        c = self.cfg
        cur, steps = self.x, []
        for l in range(self.L):
            lg = torch.empty(c.T, c.Ep, dtype=torch.float32, device=DEV)
            out = ops().mxfp4_forward_router(cur, self.w[l][0], *self.w[l][1:], c.I, c.E, c.K,
                                             c.shared, c.act_fmt, logits_out=lg)
            steps.append((cur, lg, out))
            cur = out
        torch.cuda.synchronize()
        return steps

    def oracle_layer(self, l, x_in, logits, tokens=None):
        """Layer l by the oracle on the GPU's input and fp32 logits of that layer."""
        c = self.cfg
        lg = logits.cpu().numpy()
        gate = lg[:, c.E] if c.shared else None
        ids, _ = moe.route(lg[:, :c.E], gate, c.K, c.shared)
        oracle_pack_all(synth.layer_config(c, l), np.unique(ids if tokens is None else ids[tokens]))
        return moe.forward(bits(x_in), lg[:, :c.E], gate,
                           lambda e: self.oracle_weights(l, e), c.I, c.E, c.K, c.shared,
                           c.act_fmt, tokens=tokens)


def check_layer(l, got_bits, want, act_fmt, strict=False):
    """Layer 0 (or every layer, strict) against the layer's bounds; later
    layers of an unnormalised chain with the max-abs bound per element (see
    the module's docstring)."""
    e_rel = rel_l2(got_bits, want["out"])
    if l == 0 or strict:
        e_max = max_abs_over_rms(got_bits, want)
        _say(f"  layer {l}: rel_l2 {e_rel:.2e}  max_abs/rms {e_max:.2e}")
    else:
        e_max = max_abs_elementwise(got_bits, want)
        _say(f"  layer {l}: rel_l2 {e_rel:.2e}  max_abs (per element) {e_max:.2e}")
    assert e_rel <= REL_L2[act_fmt] and e_max <= MAX_ABS_RMS


SMALL = {
    "ragged": synth.custom_config("layers_ragged", T=50, H=512, I=256, E=64, K=4, shared=1),
    "no_shared": synth.custom_config("layers_no_shared", T=33, H=256, I=128, E=24, K=2, shared=0),
    "w4a4": synth.custom_config("layers_w4a4", T=40, H=256, I=128, E=16, K=3, shared=1,
                                act_fmt=synth.ACT_MXFP4, outlier_p=0.01),
    "tiled": synth.custom_config("layers_tiled", T=300, H=512, I=256, E=16, K=3, shared=1),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_layers_match_chain_and_oracle(name):
    _say("layers", name)
    P = Layers(SMALL[name], 3)
    c = P.cfg
    steps = P.chain()
    for prefetch in (0, 1):
        out = P.multi(prefetch)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(steps[-1][2])), prefetch
    for l, (x_in, lg, out) in enumerate(steps):
        want = P.oracle_layer(l, x_in, lg)
        check_layer(l, bits(out), want, c.act_fmt)
    assert not np.array_equal(bits(steps[0][2]), bits(steps[1][2]))   # the layers differ


def test_layers_graph_replays_equal_eager():
    P = Layers(SMALL["ragged"], 2)
    c = P.cfg
    ws = torch.empty(ops().workspace_size(c.T, c.H, c.I, c.E, c.K, c.shared, c.act_fmt),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty(c.T, c.H, dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        P.multi(1, out=out, workspace=ws)
        torch.cuda.synchronize()
        eager = out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            P.multi(1, out=out, workspace=ws)
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(0)
        ws.fill_(0xFF)                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i


@pytest.mark.timeout(600)
def test_layers_full_decode():
    """Two layers of the decode workload's shapes in the configuration the
    bench times: equal to the chained calls bit for bit (with the prefetch),
    and every token of both layers against the oracle."""
    cfg = synth.CONFIGS["decode"]
    _say("layers full decode", cfg.T, cfg.H, cfg.I, cfg.E, cfg.K)
    P = Layers(cfg, 2)
    steps = P.chain()
    out = P.multi(1)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(steps[-1][2]))
    _say("  chain == multi-layer call")
    for l, (x_in, lg, got) in enumerate(steps):
        want = P.oracle_layer(l, x_in, lg)
        check_layer(l, bits(got), want, cfg.act_fmt)


# ---- the same layers with the residual add and RMSNorm after each ----------

EPS = 1e-6


def _norm_inputs(cfg, L):
    """The residual stream entering layer 0 (N(0, 1)) and each layer's norm
    weights (U(0.5, 1.5)), bf16."""
    _, r0, _ = synth.norm_inputs(1, cfg.T, cfg.H, seed=900)
    gammas = [synth.norm_inputs(1, 1, cfg.H, seed=901 + l)[2] for l in range(L)]
    return r0, gammas


def chain_norm(P, r0, gammas):
    """One call per step: the layer from its input, then the residual add and
    RMSNorm of its output.  Returns per layer (input, logits, layer output,
    residual before, residual after, normalised output) and the last residual."""
    c = P.cfg
    cur, h = P.x, r0.to(DEV).clone()
    steps = []
    for l in range(P.L):
        lg = torch.empty(c.T, c.Ep, dtype=torch.float32, device=DEV)
        y = ops().mxfp4_forward_router(cur, P.w[l][0], *P.w[l][1:], c.I, c.E, c.K, c.shared,
                                       c.act_fmt, logits_out=lg)
        h_in = h.clone()
        out, _ = ops().residual_rmsnorm([y], gammas[l].to(DEV), EPS, residual=h, residual_out=h)
        steps.append((cur, lg, y, h_in, h.clone(), out))
        cur = out
    torch.cuda.synchronize()
    return steps, h


def _multi_norm(P, r0, gammas, prefetch, **kw):
    c = P.cfg
    res = r0.to(DEV).clone()
    out = ops().mxfp4_forward_layers_norm(P.x, P.w, [g.to(DEV) for g in gammas], EPS, res, c.I,
                                          c.E, c.K, c.shared, c.act_fmt, prefetch=prefetch, **kw)
    torch.cuda.synchronize()
    return out, res


def _check_norm_steps(P, steps, gammas):
    c = P.cfg
    for l, (x_in, lg, y, h_in, h_out, out) in enumerate(steps):
        want = P.oracle_layer(l, x_in, lg)
        # every layer's input is normalised: the layer's own bounds for each
        check_layer(l, bits(y), want, c.act_fmt, strict=True)
        nd, ex = check_residual_rmsnorm(bits(y)[None], bits(h_in), bits(gammas[l]), EPS,
                                        bits(h_out), bits(out), f"norm after layer {l}")
        _say(f"  norm after layer {l}: h off by one ulp {nd}, y exact {ex:.5f}")


@pytest.mark.parametrize("name", list(SMALL))
def test_layers_norm_match_chain_and_oracle(name):
    _say("layers + residual RMSNorm", name)
    P = Layers(SMALL[name], 3)
    r0, gammas = _norm_inputs(P.cfg, 3)
    steps, h_last = chain_norm(P, r0, gammas)
    for prefetch in (0, 1):
        out, res = _multi_norm(P, r0, gammas, prefetch)
        assert np.array_equal(bits(out), bits(steps[-1][5])), prefetch
        assert np.array_equal(bits(res), bits(h_last)), prefetch
    _check_norm_steps(P, steps, gammas)


def test_layers_norm_graph_replays_equal_eager():
    P = Layers(SMALL["ragged"], 2)
    c = P.cfg
    r0, gammas = _norm_inputs(c, 2)
    g_dev = [g.to(DEV) for g in gammas]
    ws = torch.empty(ops().workspace_size(c.T, c.H, c.I, c.E, c.K, c.shared, c.act_fmt),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty(c.T, c.H, dtype=torch.bfloat16, device=DEV)
    res = torch.empty(c.T, c.H, dtype=torch.bfloat16, device=DEV)
    r0d = r0.to(DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        res.copy_(r0d)
        ops().mxfp4_forward_layers_norm(P.x, P.w, g_dev, EPS, res, c.I, c.E, c.K, c.shared,
                                        c.act_fmt, prefetch=1, out=out, workspace=ws)
        torch.cuda.synchronize()
        eager_out, eager_res = out.clone(), res.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            ops().mxfp4_forward_layers_norm(P.x, P.w, g_dev, EPS, res, c.I, c.E, c.K, c.shared,
                                            c.act_fmt, prefetch=1, out=out, workspace=ws)
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(0)
        ws.fill_(0xFF)                     # eager work between replays
        res.copy_(r0d)                     # the residual stream is updated in place
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out) and torch.equal(res, eager_res), i


@pytest.mark.timeout(600)
def test_layers_norm_full_decode():
    """Two layers of the decode workload's shapes with the residual add and
    RMSNorm after each: equal to the chained calls bit for bit, every token of
    both layers and both norm steps against the oracle."""
    cfg = synth.CONFIGS["decode"]
    _say("layers + residual RMSNorm, full decode", cfg.T, cfg.H, cfg.I, cfg.E, cfg.K)
    P = Layers(cfg, 2)
    r0, gammas = _norm_inputs(cfg, 2)
    steps, h_last = chain_norm(P, r0, gammas)
    out, res = _multi_norm(P, r0, gammas, 1)
    assert np.array_equal(bits(out), bits(steps[-1][5]))
    assert np.array_equal(bits(res), bits(h_last))
    _say("  chain == multi-layer call")
    _check_norm_steps(P, steps, gammas)
