"""moe_residual_rmsnorm on the GPU against the oracle: the ranks' partial
outputs summed, the residual added, RMSNorm (VibeSys "Qwen3.5-397B on 4x
MI300A" post, section "Communication and concurrency": the all-reduce fused
with the residual add and RMSNorm), element by element on every output.

Shapes: the decode batch at tensor-parallel degree 8 (T = 64, H = 4096,
eight partials), the 1,536-token prefill chunk and the 8,192-token one
(whose inputs exceed the memory-side cache and take the non-temporal loads);
H = 6144, 8192 and 16384 (the kernel's three, four and eight column groups
per thread, the last fetching group by group); a ragged H that leaves most
threads idle; one rank; no residual; in-place updates of the residual stream
and of partial 0; rows of zeros, of values near eps, and of large values."""
import sys

import numpy as np
import pytest
import torch

import synth
from tests.helpers import DEV, bits, check_residual_rmsnorm

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    # name: (G, T, H, eps, with residual)
    "one_rank_tiny": (1, 1, 8, 1e-6, True),
    "ragged_h136": (3, 5, 136, 1e-6, True),
    "no_residual": (2, 7, 2048, 1e-5, False),
    "decode_tp8": (8, 64, 4096, 1e-6, True),
    "h6144_tp4": (4, 33, 6144, 1e-6, True),
    "h8192_tp2": (2, 9, 8192, 1e-6, True),
    "h16384_tp8": (8, 3, 16384, 1e-6, True),
    "prefill_tp8": (8, 1536, 4096, 1e-6, True),
    # inputs above the memory-side cache (590 MB): the non-temporal loads
    "prefill_skewed_tp8": (8, 8192, 4096, 1e-6, True),
}


def _run(p, r, g, eps, inplace=False):
    from mxfp4_routed_expert_top_amd import ops
    parts = [p[i].to(DEV).contiguous() for i in range(p.shape[0])]
    res = None if r is None else r.to(DEV).contiguous()
    gam = g.to(DEV)
    if inplace:
        # the residual stream updated in place, the output over partial 0
        out, hout = ops.residual_rmsnorm(parts, gam, eps, residual=res, residual_out=res,
                                         out=parts[0])
    else:
        hout = torch.empty_like(parts[0])
        out, _ = ops.residual_rmsnorm(parts, gam, eps, residual=res, residual_out=hout)
    torch.cuda.synchronize()
    return bits(hout.cpu()), bits(out.cpu())


@pytest.mark.parametrize("name", list(CASES))
def test_residual_rmsnorm_matches_the_oracle(name):
    G, T, H, eps, with_res = CASES[name]
    _say("residual_rmsnorm", name, "G", G, "T", T, "H", H)
    p, r, g = synth.norm_inputs(G, T, H, seed=101 + G * 7 + H)
    if not with_res:
        r = None
    h, y = _run(p, r, g, eps)
    nd, ex = check_residual_rmsnorm(bits(p), None if r is None else bits(r), bits(g), eps, h, y,
                                    name)
    _say(f"  {name}: h elements off by one ulp {nd}, y exactly rounded {ex:.5f}")


def test_residual_rmsnorm_in_place():
    G, T, H, eps = 4, 16, 4096, 1e-6
    p, r, g = synth.norm_inputs(G, T, H, seed=7)
    h, y = _run(p, r, g, eps, inplace=True)
    check_residual_rmsnorm(bits(p), bits(r), bits(g), eps, h, y, "in place")
    # the same bits as the out-of-place call
    h2, y2 = _run(p, r, g, eps)
    assert np.array_equal(h, h2) and np.array_equal(y, y2)


def test_residual_rmsnorm_special_rows():
    # zeros (rstd = 1/sqrt(eps)), a row whose mean square is near eps, a row
    # of large values, a row with one large element among small ones
    G, T, H, eps = 2, 4, 4096, 1e-6
    p = torch.zeros(G, T, H, dtype=torch.float32)
    r = torch.zeros(T, H, dtype=torch.float32)
    r[1] = 2.0 ** -10
    p[0, 1, ::3] = 2.0 ** -11
    r[2] = 2.0 ** 50
    p[1, 2, 1::2] = -(2.0 ** 49)
    r[3] = 1e-3
    r[3, 17] = 300.0
    g = torch.linspace(0.5, 1.5, H)
    pb, rb, gb = p.to(torch.bfloat16), r.to(torch.bfloat16), g.to(torch.bfloat16)
    h, y = _run(pb, rb, gb, eps)
    check_residual_rmsnorm(bits(pb), bits(rb), bits(gb), eps, h, y, "special rows")
    assert not np.any(y[0]), "a zero row normalises to zeros"


def test_residual_rmsnorm_empty_batch():
    from mxfp4_routed_expert_top_amd import ops
    parts = [torch.empty(0, 4096, dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    gam = torch.ones(4096, dtype=torch.bfloat16, device=DEV)
    out, _ = ops.residual_rmsnorm(parts, gam, 1e-6)
    torch.cuda.synchronize()
    assert out.shape == (0, 4096)
