"""Shared set-up of the GPU parity tests: seeded inputs (synth), weights
packed once by the GPU path's quantiser and once by the oracle's, and the
comparison measures the layer's tolerances are stated in."""
from __future__ import annotations

import functools

import numpy as np
import torch

import synth
from oracle import moe, mxfp4

DEV = "cuda"

# Tolerances of the bf16 output against the oracle (relative L2 error; and
# max-abs error relative to the oracle output's RMS).
REL_L2 = {synth.ACT_BF16: 5e-3, synth.ACT_MXFP4: 2e-2}
MAX_ABS_RMS = 2e-2
W_ATOL = 1e-6          # routing weights, absolute


def native_order(codes: np.ndarray, nq: int) -> np.ndarray:
    """Row-major weight codes [rows, row_bytes] -> the GEMM kernels' native
    code order (the permutation include/moe_mxfp4.h defines), by reshapes:
    row 16 s + n, byte nq (64 c + 16 g) + 16 q + b  ->  block (s, c, q),
    lane 16 g + n, byte b.  nq = 1 (MXFP4) or 2 (MXFP8)."""
    rows, rb = codes.shape
    C = rb // (64 * nq)
    a = codes.reshape(rows // 16, 16, C, 4, nq, 16)      # s, n, c, g, q, b
    return np.ascontiguousarray(a.transpose(0, 2, 4, 3, 1, 5)).reshape(rows, rb)


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


def max_abs_over_rms(got_bits, want_bits) -> float:
    g = mxfp4.bf16_to_f64(got_bits)
    w = mxfp4.bf16_to_f64(want_bits)
    rms = float(np.sqrt(np.mean(w * w)))
    return float(np.max(np.abs(g - w)) / max(rms, 1e-300))


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

    @functools.lru_cache(maxsize=None)
    def oracle_weights(self, e: int):
        """Expert e packed by the oracle's own quantiser from the same draws."""
        c = self.cfg
        a = mxfp4.quantize(synth.expert_w13(c, e, DEV).cpu().numpy())
        b = mxfp4.quantize(synth.expert_w2(c, e, DEV).cpu().numpy())
        return a[0], a[1], b[0], b[1]

    def oracle(self, tokens=None, act_fmt=None):
        c = self.cfg
        return moe.forward(bits(self.x_cpu), self.logits_cpu.numpy(),
                           None if self.gate_cpu is None else self.gate_cpu.numpy(),
                           self.oracle_weights, c.I, c.E, c.K, c.shared,
                           c.act_fmt if act_fmt is None else act_fmt, tokens=tokens)

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
