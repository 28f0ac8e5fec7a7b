"""Shared set-up of the GPU parity tests: seeded inputs (synth), weights
packed once by the GPU path's quantiser and once by the oracle's, and the
comparison measures the layer's tolerances are stated in."""
from __future__ import annotations

import numpy as np
import torch

import synth
from oracle import moe, mxfp4, mxfp8

DEV = "cuda"

# Tolerances of the bf16 output against the oracle (relative L2 error; and
# max-abs error relative to the oracle output's RMS).
REL_L2 = {synth.ACT_BF16: 5e-3, synth.ACT_MXFP4: 2e-2}
MAX_ABS_RMS = 2e-2
W_ATOL = 1e-6          # routing weights, absolute


def native_order(codes: np.ndarray, nq: int) -> np.ndarray:
    """Row-major weight codes [rows, row_bytes] -> the GEMM kernels' native
    code order (the permutation include/moe_mxfp4.h defines), by reshapes:
    row 32 p + 8 a + 4 u + b, byte nq (64 c + 16 g) + 16 q + j  ->  block
    (s = 2 p + u, c, q), lane 16 g + 4 a + b, byte j.  nq = 1 (MXFP4) or 2
    (MXFP8)."""
    rows, rb = codes.shape
    C = rb // (64 * nq)
    a = codes.reshape(rows // 32, 4, 2, 4, C, 4, nq, 16)   # p, a, u, b, c, g, q, j
    return np.ascontiguousarray(a.transpose(0, 2, 4, 6, 5, 1, 3, 7)).reshape(rows, rb)


def blocked_order(codes: np.ndarray, scales: np.ndarray):
    """Row-major MXFP4 activations (codes [R, cols/2], scales [R, cols/32],
    R a multiple of 16) -> the blocked row order of include/moe_mxfp4.h
    (moe_mxfp4_quantize_blocked), by reshapes: row 16 b + n, chunk c ->
    codes block (b, c) byte 64 n + j, scales block (b, c) byte 4 n + g."""
    R, cb = codes.shape
    C = cb // 64
    pc = codes.reshape(R // 16, 16, C, 64).transpose(0, 2, 1, 3)
    ps = scales.reshape(R // 16, 16, C, 4).transpose(0, 2, 1, 3)
    return (np.ascontiguousarray(pc).reshape(R, cb),
            np.ascontiguousarray(ps).reshape(R, scales.shape[1]))


def unblocked_rows(codes: np.ndarray, scales: np.ndarray):
    """The inverse of blocked_order: blocked MXFP4 activations -> row-major rows."""
    R, cb = codes.shape
    C = cb // 64
    rc = codes.reshape(R // 16, C, 16, 64).transpose(0, 2, 1, 3).reshape(R, cb)
    rs = scales.reshape(R // 16, C, 16, 4).transpose(0, 2, 1, 3).reshape(R, scales.shape[1])
    return rc, rs


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 numpy bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def rel_l2(got_bits, want_bits) -> float:
    g = mxfp4.bf16_to_f64(got_bits)
    w = mxfp4.bf16_to_f64(want_bits)
    return float(np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-300))


def max_abs_over_rms(got_bits, want) -> float:
    """Max-abs error of a bf16 output over the RMS of the reference output.

    want = the oracle's result dict: the error is measured against the
    oracle's fp64 output before its own final rounding (out_f64), beyond the
    half bf16 spacing by which the GPU output itself is rounded:
    max_j(|got_j - out_f64_j| - ulp(got_j) / 2) / RMS.  A bf16 output cannot
    come closer to the exact value than its own rounding, and above ~5 x RMS
    half a spacing alone exceeds 1% of the RMS, so the layer's bound
    (2e-2 x RMS) applies to the error beyond it.  This is the plain
    |got - want_bits| bound with at most one output ulp of slack.
    want = bf16 bits (a GPU-vs-GPU comparison): plain max |got - want|."""
    g = mxfp4.bf16_to_f64(got_bits)
    if isinstance(want, dict):
        w = mxfp4.bf16_to_f64(want["out"])
        f = np.asarray(want["out_f64"], dtype=np.float64)
        rms = float(np.sqrt(np.mean(w * w)))
        err = np.maximum(np.abs(g - f) - 0.5 * bf16_ulp(g), 0.0)
        return float(np.max(err) / max(rms, 1e-300)) if err.size else 0.0
    w = mxfp4.bf16_to_f64(want)
    rms = float(np.sqrt(np.mean(w * w)))
    return float(np.max(np.abs(g - w)) / max(rms, 1e-300))


def say(*a):
    print(*a, flush=True)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (2^(e-7) for |v| in [2^e, 2^(e+1));
    the subnormal spacing 2^-133 at zero)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, ex = np.frexp(v)
    return np.where(v == 0, 2.0 ** -133, np.ldexp(1.0, np.maximum(ex - 8, -133)))


def diff_report(got_bits, want_bits, want_f64=None) -> dict:
    """Where two bf16 outputs differ: in units of bf16 spacing (ulp) at the
    oracle's value, and where the largest differences sit relative to RMS."""
    g, w = mxfp4.bf16_to_f64(got_bits), mxfp4.bf16_to_f64(want_bits)
    rms = float(np.sqrt(np.mean(w * w)))
    d = np.abs(g - w)
    ulps = d / bf16_ulp(np.maximum(np.abs(w), np.abs(g)))
    j = int(np.argmax(d))
    rep = {"rms": rms, "max_over_rms_of_want": float(np.max(np.abs(w)) / rms),
           "worst": {"index": np.unravel_index(j, d.shape), "got": float(g.flat[j]),
                     "want": float(w.flat[j]), "want_over_rms": float(abs(w.flat[j]) / rms),
                     "ulps": float(ulps.flat[j])},
           "ulps_hist": {"0": int((ulps == 0).sum()), "1": int((ulps == 1).sum()),
                         "2": int((ulps == 2).sum()), ">2": int((ulps > 2).sum())},
           "over_2e-2_rms": int((d > 2e-2 * rms).sum()),
           "max_ulps": float(ulps.max())}
    big = ulps > 1
    rep["max_abs_over_rms_beyond_1ulp"] = float(d[big].max() / rms) if big.any() else 0.0
    if want_f64 is not None:
        e = np.abs(g - want_f64)
        rep["max_abs_vs_f64_over_rms"] = float(e.max() / rms)
        rep["max_excess_over_half_ulp_over_rms"] = float(
            np.max(e - 0.5 * bf16_ulp(g)) / rms)
    return rep


# Expert weights packed by the oracle's own quantiser, shared by every test
# of a session (the full-size workloads reuse one draw): key = the draw and
# the format.
_ORACLE_WEIGHTS: dict = {}


def oracle_pack(cfg: synth.MoEConfig, e: int, wfmt: int = synth.W_MXFP4):
    """Expert e of cfg's weight draw packed by the oracle's quantiser (the same
    float tensors the GPU path packs, drawn on the GPU and copied)."""
    key = (cfg.seed_w, cfg.H, cfg.I, cfg.w_std, wfmt, e)
    if key not in _ORACLE_WEIGHTS:
        q = mxfp8.quantize if wfmt == synth.W_MXFP8 else mxfp4.quantize
        a = q(synth.expert_w13(cfg, e, DEV).cpu().numpy())
        b = q(synth.expert_w2(cfg, e, DEV).cpu().numpy())
        _ORACLE_WEIGHTS[key] = (a[0], a[1], b[0], b[1])
    return _ORACLE_WEIGHTS[key]


def oracle_pack_all(cfg: synth.MoEConfig, experts, wfmt: int = synth.W_MXFP4) -> None:
    """Pack the listed experts ahead of an oracle call, printing progress."""
    experts = [int(e) for e in experts]
    for i, e in enumerate(experts):
        if i % 128 == 0:
            say(f"  oracle packing expert {i}/{len(experts)}")
        oracle_pack(cfg, e, wfmt)


class Problem:
    """One workload on the GPU plus lazy oracle-side weights."""

    def __init__(self, cfg: synth.MoEConfig, logits=None):
        from mxfp4_routed_expert_top_amd import ops
        self.cfg = cfg
        c = cfg
        self.x_cpu = synth.activations(c)
        self.logits_cpu = synth.router_logits(c) if logits is None else logits
        self.gate_cpu = synth.gate_logits(c)
        self.x = self.x_cpu.to(DEV)
        self.logits = self.logits_cpu.to(DEV)
        self.gate = None if self.gate_cpu is None else self.gate_cpu.to(DEV)
        u8 = dict(dtype=torch.uint8, device=DEV)
        self.w13 = torch.empty(c.Ep, 2 * c.I, c.H // 2, **u8)
        self.w13s = torch.empty(c.Ep, 2 * c.I, c.H // 32, **u8)
        self.w2 = torch.empty(c.Ep, c.H, c.I // 2, **u8)
        self.w2s = torch.empty(c.Ep, c.H, c.I // 32, **u8)
        for e in range(c.Ep):
            ops.quantize_weights(synth.expert_w13(c, e, DEV), self.w13[e], self.w13s[e])
            ops.quantize_weights(synth.expert_w2(c, e, DEV), self.w2[e], self.w2s[e])
        torch.cuda.synchronize()

    def oracle_weights(self, e: int):
        """Expert e packed by the oracle's own quantiser from the same draws."""
        return oracle_pack(self.cfg, e)

    def oracle(self, tokens=None, act_fmt=None, return_h=False):
        """The oracle's layer on the same inputs (every token unless `tokens`);
        the experts it needs are packed first, with progress lines."""
        c = self.cfg
        logits = self.logits_cpu.numpy()
        gate = None if self.gate_cpu is None else self.gate_cpu.numpy()
        ids, _ = moe.route(logits, gate, c.K, c.shared)
        sel = ids if tokens is None else ids[np.asarray(tokens)]
        oracle_pack_all(c, np.unique(sel))
        return moe.forward(bits(self.x_cpu), logits, gate, self.oracle_weights, c.I, c.E, c.K,
                           c.shared, c.act_fmt if act_fmt is None else act_fmt, tokens=tokens,
                           return_h=return_h)

    def forward(self, **kw):
        from mxfp4_routed_expert_top_amd import ops
        c = self.cfg
        return ops.mxfp4_forward(self.x, self.logits, self.gate, self.w13, self.w13s, self.w2,
                                 self.w2s, c.I, c.E, c.K, c.shared, c.act_fmt, **kw)

    def stages(self, **kw):
        from mxfp4_routed_expert_top_amd import ops
        c = self.cfg
        return ops.forward_stages(self.x, self.logits, self.gate, self.w13, self.w13s, self.w2,
                                  self.w2s, c.I, c.E, c.K, c.shared, c.act_fmt, **kw)


def check_residual_rmsnorm(p_bits, r_bits, g_bits, eps, h_gpu, y_gpu, what=""):
    """The kernel's h and y (bf16 bits) against the oracle on the same inputs.

    h: the kernel sums residual and partials in fp32, the oracle in fp64; for
    bf16 inputs the fp32 sum is exact unless their exponents span more than
    16 bits, and even then its bf16 rounding changes only when the sum lies
    within an fp32 rounding of a bf16 midpoint.  So h must be equal, with at
    most one element in 10^4 one bf16 ulp away.
    y: the kernel's fp32 mean of squares, reciprocal square root and two
    products carry a relative error of a few times 1e-7 (up to H * 2^-24 for
    the sum), far below half a bf16 ulp (2^-9), so its bf16 y is one of the
    two bf16 neighbours of the exact y = h * rstd * gamma: |y - y_exact| <=
    one bf16 ulp of y_exact, and exact rounding almost everywhere (>= 99%).
    Elements whose h differed are left out of the y check."""
    want_h, _, rstd = moe.residual_rmsnorm(p_bits, r_bits, g_bits, eps)
    hg, hw = mxfp4.bf16_to_f64(h_gpu), mxfp4.bf16_to_f64(want_h)
    diff = hg != hw
    n = hw.size
    assert diff.sum() <= max(0, n // 10000), f"{what}: {diff.sum()} h elements differ"
    if diff.any():
        assert np.all(np.abs(hg[diff] - hw[diff]) <= bf16_ulp(hw[diff])), f"{what}: h off by > 1 ulp"
    gam = mxfp4.bf16_to_f64(g_bits)
    y_exact = hw * rstd[:, None] * gam[None, :]
    yg = mxfp4.bf16_to_f64(y_gpu)
    ok = ~diff
    zero = ok & (y_exact == 0)
    assert np.all(yg[zero] == 0), f"{what}: y of a zero h is not zero"
    nz = ok & (y_exact != 0)
    err = np.abs(yg[nz] - y_exact[nz])
    assert np.all(err <= bf16_ulp(y_exact[nz])), f"{what}: y off by more than one bf16 ulp"
    exact = np.mean(y_gpu[ok] == mxfp4.bf16_bits(y_exact[ok]))
    assert exact >= 0.99, f"{what}: only {exact:.4f} of y rounded exactly"
    return int(diff.sum()), float(exact)
