"""What one GPU can show of a tensor-parallel split of the layer.

With G GPUs each holding every expert's I/G slice (gate rows, up rows and
down columns) and the routing replicated, the layer's output is the sum of
the G shard layers' outputs (the all-reduce the split would need).  Here the
G shard layers run one after another on one GPU, from slices of the same
packed weights: routing must be identical, each shard's h must be the exact
column slice of the full layer's h, each shard's output must match the
oracle's layer on the same weight slices (the layer's tolerance), and the
sum of the shards' outputs must match the full layer.  The step that
follows the layer in such a split, the ranks' outputs summed with the
residual added and RMSNorm applied (moe_residual_rmsnorm, the epilogue of
the pages' one-shot all-reduce), then runs on the G shard outputs with x as
the residual stream and is checked against the oracle on the same bits.

The sum carries roundings the single layer does not: each shard rounds its
own y and out to bf16 (relative error <= 2^-9 each), and the shards' parts
can be larger than their sum.  The identity is checked as rel-L2 <= 1e-2
(about sqrt(G) x 2 x 2^-9 x the parts-to-sum RMS ratio, with margin) and
max-abs <= 5e-2 x RMS; the parity proper is the per-shard comparison."""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import moe
from tests.helpers import (DEV, MAX_ABS_RMS, REL_L2, W_ATOL, Problem, bits,
                           check_residual_rmsnorm, max_abs_over_rms, oracle_pack_all, rel_l2)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _shard(prob, g, G):
    """Expert weights of shard g of G: I/G gate rows, I/G up rows, I/G down
    columns, sliced from the row-major packing of the same draws (the
    library's quantiser), then put into the native code order."""
    from mxfp4_routed_expert_top_amd import ops
    c = prob.cfg
    Ig = c.I // G
    rows = torch.cat([torch.arange(g * Ig, (g + 1) * Ig), torch.arange(c.I + g * Ig, c.I + (g + 1) * Ig)]).to(DEV)
    u8 = dict(dtype=torch.uint8, device=DEV)
    w13 = torch.empty(c.Ep, 2 * Ig, c.H // 2, **u8)
    w13s = torch.empty(c.Ep, 2 * Ig, c.H // 32, **u8)
    w2 = torch.empty(c.Ep, c.H, Ig // 2, **u8)
    w2s = torch.empty(c.Ep, c.H, Ig // 32, **u8)
    for e in range(c.Ep):
        q, s = ops.mxfp4_quantize(synth.expert_w13(c, e, DEV))
        ops.weights_to_native(q.index_select(0, rows).contiguous(), out=w13[e])
        w13s[e] = s.index_select(0, rows)
        q, s = ops.mxfp4_quantize(synth.expert_w2(c, e, DEV))
        ops.weights_to_native(q[:, g * Ig // 2:(g + 1) * Ig // 2].contiguous(), out=w2[e])
        w2s[e] = s[:, g * Ig // 32:(g + 1) * Ig // 32]
    return w13, w13s, w2, w2s, Ig


CASES = {
    "tp4_small": (synth.custom_config("tp4_small", T=50, H=512, I=512, E=64, K=4, shared=1), 4),
    "tp4_tiled": (synth.custom_config("tp4_tiled", T=300, H=512, I=512, E=16, K=3, shared=1), 4),
    "tp2_w4a4": (synth.custom_config("tp2_w4a4", T=40, H=256, I=256, E=16, K=3, shared=1,
                                     act_fmt=synth.ACT_MXFP4, outlier_p=0.01), 2),
    "tp8_decode": (synth.CONFIGS["decode"], 8),
}


@pytest.mark.parametrize("name", list(CASES))
def test_tensor_parallel_shards_sum_to_the_layer(name):
    from mxfp4_routed_expert_top_amd import ops
    cfg, G = CASES[name]
    _say("tp shards", name, "G", G)
    prob = Problem(cfg)
    c = cfg
    full = prob.stages()
    torch.cuda.synchronize()
    tokens = None                      # every token against the oracle
    oracle_pack_all(c, np.unique(full["ids"].cpu().numpy()))
    acc = torch.zeros(c.T, c.H, dtype=torch.float32, device=DEV)
    outs = []
    for g in range(G):
        w13, w13s, w2, w2s, Ig = _shard(prob, g, G)
        r = ops.forward_stages(prob.x, prob.logits, prob.gate, w13, w13s, w2, w2s, Ig, c.E, c.K,
                               c.shared, c.act_fmt)
        torch.cuda.synchronize()
        assert torch.equal(r["ids"], full["ids"]) and torch.equal(r["w"], full["w"])
        if r["align"]["tile_m"] == full["align"]["tile_m"]:
            # each output column of gate/up + SwiGLU sums over K in the same order
            assert torch.equal(r["h"], full["h"][:, g * Ig:(g + 1) * Ig])
        acc += r["out"].float()
        outs.append(r["out"].clone())
        if g < 2:                      # the oracle's layer on this shard's weight slices
            Ig2, b2, s2 = Ig, Ig // 2, Ig // 32

            def wsh(e, g=g):
                w13, w13s, w2, w2s = prob.oracle_weights(e)
                rows = np.r_[g * Ig2:(g + 1) * Ig2, c.I + g * Ig2:c.I + (g + 1) * Ig2]
                return (w13[rows], w13s[rows], w2[:, g * b2:(g + 1) * b2],
                        w2s[:, g * s2:(g + 1) * s2])
            want = moe.forward(bits(prob.x_cpu), prob.logits_cpu.numpy(),
                               None if prob.gate_cpu is None else prob.gate_cpu.numpy(), wsh,
                               Ig, c.E, c.K, c.shared, c.act_fmt, tokens=tokens)
            got = bits(r["out"]) if tokens is None else bits(r["out"])[tokens]
            e_rel, e_max = rel_l2(got, want["out"]), max_abs_over_rms(got, want)
            _say(f"  shard {g}: vs the oracle on its slices: rel_l2 {e_rel:.2e}  max_abs/rms {e_max:.2e}")
            assert e_rel <= REL_L2[c.act_fmt] and e_max <= MAX_ABS_RMS
    got, ref = bits(acc.to(torch.bfloat16)), bits(full["out"])
    e_rel, e_max = rel_l2(got, ref), max_abs_over_rms(got, ref)
    _say(f"  {name}: sum of {G} shards vs the full layer: rel_l2 {e_rel:.2e}  max_abs/rms {e_max:.2e}")
    assert e_rel <= 1e-2 and e_max <= 5e-2
    # the fused epilogue of the all-reduce: shard outputs + x, RMSNorm
    _, _, gamma = synth.norm_inputs(1, 1, c.H, seed=11)
    hres = torch.empty_like(prob.x)
    y, _ = ops.residual_rmsnorm(outs, gamma.to(DEV), 1e-6, residual=prob.x, residual_out=hres)
    torch.cuda.synchronize()
    nd, ex = check_residual_rmsnorm(np.stack([bits(o) for o in outs]), bits(prob.x_cpu),
                                    bits(gamma), 1e-6, bits(hres), bits(y), name)
    _say(f"  {name}: residual + sum of shards, RMSNorm: h off by one ulp {nd}, y exact {ex:.5f}")
