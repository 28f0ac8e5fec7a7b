"""The no-allocation forward (moe_mxfp4_forward_noalloc, the library's own
device scratch instead of a workspace) against moe_mxfp4_forward on the same
inputs: bit for bit, on consecutive calls of different sizes (the scratch
keeps the previous call's contents), W4A16 and W4A4, the 32-row and the
LDS-tiled kernels; a call beyond the scratch's limit is rejected before it
touches its outputs."""
import sys

import numpy as np
import pytest
import torch

import synth
from tests.helpers import DEV, Problem, bits

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ops():
    from mxfp4_routed_expert_top_amd import ops as o
    return o


def _both(prob, T=None):
    """(noalloc output, ids, weights), (forward output, ids, weights) on the
    first T tokens of the problem."""
    c = prob.cfg
    T = c.T if T is None else T
    x, lg = prob.x[:T].contiguous(), prob.logits[:T].contiguous()
    g = None if prob.gate is None else prob.gate[:T].contiguous()
    res = []
    for fn in (ops().mxfp4_forward_noalloc, ops().mxfp4_forward):
        ids = torch.full((T, c.Kp), -1, dtype=torch.int32, device=DEV)
        w = torch.full((T, c.Kp), -1.0, dtype=torch.float32, device=DEV)
        out = fn(x, lg, g, prob.w13, prob.w13s, prob.w2, prob.w2s, c.I, c.E, c.K, c.shared,
                 c.act_fmt, topk_ids=ids, topk_weights=w)
        torch.cuda.synchronize()
        res.append((bits(out), ids.cpu().numpy(), w.cpu().numpy()))
    return res


@pytest.mark.parametrize("act", [synth.ACT_BF16, synth.ACT_MXFP4])
def test_noalloc_forward_equals_forward_on_consecutive_calls(act):
    cfg = synth.custom_config("noalloc", T=300, H=512, I=256, E=16, K=3, shared=1, act_fmt=act,
                              outlier_p=0.002 if act else 0.0)
    prob = Problem(cfg)
    o = ops()
    for T in (300, 40, 7):         # tiled GEMMs, then the 32-row kernels, then a tiny batch
        tm = o.gemm_tile_m(T, cfg.Kp, cfg.Ep, cfg.H, cfg.I, act)
        (na, na_ids, na_w), (fw, fw_ids, fw_w) = _both(prob, T)
        _say(f"  act {act} T {T} tile_m {tm}: identical {np.array_equal(na, fw)}")
        assert np.array_equal(na, fw)
        assert np.array_equal(na_ids, fw_ids) and np.array_equal(na_w, fw_w)


def test_noalloc_decode_shape_and_limit():
    cfg = synth.CONFIGS["decode"]
    prob = Problem(cfg)
    (na, _, _), (fw, _, _) = _both(prob)
    assert np.array_equal(na, fw)
    (na, _, _), (fw, _, _) = _both(prob, 17)          # smaller, after the full batch
    assert np.array_equal(na, fw)
    # beyond the scratch (588 decode tokens): rejected, outputs untouched
    c = cfg
    T = 588
    assert ops().workspace_size(T, c.H, c.I, c.E, c.K, c.shared, c.act_fmt) > ops().NOALLOC_SCRATCH_BYTES
    x = torch.zeros(T, c.H, dtype=torch.bfloat16, device=DEV)
    lg = torch.zeros(T, c.E, dtype=torch.float32, device=DEV)
    g = torch.zeros(T, dtype=torch.float32, device=DEV)
    out = torch.full((T, c.H), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ops().MoeError) as ei:
        ops().mxfp4_forward_noalloc(x, lg, g, prob.w13, prob.w13s, prob.w2, prob.w2s, c.I, c.E,
                                    c.K, c.shared, c.act_fmt, out=out)
    assert ei.value.status == ops().MOE_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert bool((out.float() == 7.0).all())
