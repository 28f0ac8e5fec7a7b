"""The MXFP4 routed-expert MoE layer computed from its plain definition
(fp64): Python access to the C++ oracle (oracle/moe_oracle.cpp).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package.  It shares no code with the HIP
path and never imports it.  This module only marshals arrays and picks the
experts a call needs; the arithmetic is the C++ oracle's.

What the layer computes, per token t with router logits l_t, activations
x_t and (when the shared expert is folded in) gate logit g_t:

  S_t   = the K experts with the largest logits, ties to the lower index
          (softmax is monotone, so this is top-K of the softmax scores;
          InferenceX "MI355X Qwen3.5 SGLang v0.5.12" post, section on the
          specific optimisations, fused_topk bullet: softmax-scored top-K
          at E=512, K=10)
  w_t,e = softmax(l_t)_e / sum_{e' in S_t} softmax(l_t)_e'  (renormalised)
  the shared expert is one more expert, index E, in slot K, with weight
          sigmoid(g_t) (same post, shared-expert fusion bullet: the shared
          expert becomes expert top-K+1 of one MoE dispatch; MiniMax M3 on
          MI355X post, section "Shared expert fusion")
  MLP_e(a) = W2_e . bf16( silu(W13_e[gate] . a) * (W13_e[up] . a) )
  out_t = bf16( sum_k w_t,k * MLP_{e_k}(x_t) ), summed in slot order.

MXFP4 weights are decoded exactly; each dot product is an fp64 sum of exact
products; bf16 rounding happens where the GPU path stores bf16: h, out,
and (round_y) each slot's expert output y where a path stages it in bf16
between the down GEMM and the combine (the pages fix no precision for y).
For W4A4 the activations and h are MXFP4-quantised then decoded before
their GEMM (OpenRelay "Gemma 4 31B on MI355X" post, sections
"Optimisation 3" and "Optimisation 4": activation + MXFP4 quantisation
fused into one kernel).

Grouping by expert (align) is a stable sort of the flat assignment ids
t*K'+k by expert id; the tile list is the tile_m-row tiles of each
expert's group (VibeSys post, section "Prefill, cache and speculation":
32-row tiles in the MoE kernel).

The router GEMM that produces the logits (the step before routing; the
InferenceX post's fused_topk consumes a separately computed gating output)
is logits = x . Wr^T over bf16 x and bf16 router rows, and with a shared
expert the gate logit g = x . Wr[E] of one more row: router_logits computes
it in fp64 over exact products.

Expert weights may also be MXFP8 (oracle/mxfp8.py), with bf16 activations;
everything else is unchanged.

After the layer, a tensor-parallel decode sums the ranks' partial outputs,
adds the residual stream and applies RMSNorm in one step (VibeSys post,
section "Communication and concurrency": the all-reduce replaced by a
one-shot one fused with the residual add and RMSNorm): residual_rmsnorm,
with RMSNorm in its textbook form (the pages do not define it).

Pins: tests/test_oracle_moe.py, tests/golden/route_align.json,
tests/golden/w4a4_worked.json.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import mxfp4, mxfp8
from ._lib import check, default_threads, lib, ptr

ACT_BF16 = 0
ACT_MXFP4 = 1
# expert weight formats: MXFP4 (two E2M1 codes per byte) or MXFP8 (one E4M3
# code per byte), both with one E8M0 scale per 32 elements along K
W_MXFP4 = 0
W_MXFP8 = 1


def decode_weights(codes, scales, wfmt: int) -> np.ndarray:
    """Expert weight rows -> fp64, exact, in either format."""
    return mxfp8.decode(codes, scales) if wfmt == W_MXFP8 else mxfp4.decode(codes, scales)


def route(logits: np.ndarray, gate, K: int, shared: int, renormalize: bool = True):
    """Softmax top-K routing.

    logits fp32 [T, E]; gate fp32 [T] (used when shared == 1).
    Returns ids int32 [T, K+shared] and weights fp32 [T, K+shared].
    Slots 0..K-1 hold the routed experts ordered by (logit descending,
    index ascending); -0.0 and +0.0 compare equal.  Weights are computed in
    fp64 and rounded to fp32:
      renormalised: exp(l_k - l_max) / sum_{k' < K} exp(l_k' - l_max)
      otherwise:    exp(l_k - l_max) / sum_{all e} exp(l_e - l_max)
    Slot K (shared): id E, weight 1 / (1 + exp(-g))."""
    l = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = l.shape
    Kp = K + shared
    g = np.ascontiguousarray(gate, dtype=np.float32) if shared else None
    ids = np.empty((T, Kp), dtype=np.int32)
    w = np.empty((T, Kp), dtype=np.float32)
    check(lib().oracle_route(ptr(l), ptr(g), T, E, K, shared, int(bool(renormalize)), ptr(ids),
                             ptr(w)), "route")
    return ids, w


def residual_rmsnorm(partials_bits: np.ndarray, residual_bits, gamma_bits: np.ndarray,
                     eps: float):
    """Partial outputs bf16 bits [G, T, H] summed, the residual [T, H] (bf16
    bits, or None for zeros) added, then RMSNorm with gamma [H] (bf16 bits):
    h = bf16(residual + sum_g partial_g) (fp64 sums of exact values),
    y = bf16(h / sqrt(mean_j h^2 + eps) * gamma).  Returns (h bits, y bits,
    rstd fp64 [T])."""
    p = np.ascontiguousarray(partials_bits, dtype=np.uint16)
    G, T, H = p.shape
    gm = np.ascontiguousarray(gamma_bits, dtype=np.uint16)
    assert gm.shape == (H,)
    r = None if residual_bits is None else np.ascontiguousarray(residual_bits, dtype=np.uint16)
    assert r is None or r.shape == (T, H)
    h = np.empty((T, H), dtype=np.uint16)
    y = np.empty((T, H), dtype=np.uint16)
    rstd = np.empty(T, dtype=np.float64)
    check(lib().oracle_residual_rmsnorm(ptr(p), G, None if r is None else ptr(r), ptr(gm),
                                        float(eps), T, H, ptr(h), ptr(y), ptr(rstd)),
          "residual_rmsnorm")
    return h, y, rstd


def router_logits(x_bits: np.ndarray, w_bits: np.ndarray, threads: int | None = None) -> np.ndarray:
    """Router GEMM: x bf16 bits [T, H], router rows bf16 bits [R, H] ->
    fp64 [T, R] = x . W^T.  The inputs are decoded exactly and each product
    of two bf16 values is exact in fp64; the sums are fp64."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    wr = np.ascontiguousarray(w_bits, dtype=np.uint16)
    T, H = x.shape
    R = wr.shape[0]
    assert wr.shape[1] == H
    out = np.empty((T, R), dtype=np.float64)
    check(lib().oracle_router_logits(ptr(x), ptr(wr), T, R, H, ptr(out),
                                     threads or default_threads()), "router_logits")
    return out


def align(ids: np.ndarray, Ep: int, tile_m: int = 32):
    """Group the flat assignments a = t*K'+k by expert, stably.

    Returns counts int32 [Ep], offsets int32 [Ep+1] (exclusive scan, the
    last entry = A), sorted int32 [A] (flat ids grouped by expert,
    ascending inside a group), inv int32 [A] (position of each flat id in
    sorted), tiles int32 [n_tiles, 2] (expert, first row) for tile_m-row
    tiles, expert-major and ascending, and n_tiles."""
    flat = np.ascontiguousarray(np.asarray(ids).reshape(-1), dtype=np.int32)
    A = flat.size
    counts = np.empty(Ep, dtype=np.int32)
    offsets = np.empty(Ep + 1, dtype=np.int32)
    srt = np.empty(A, dtype=np.int32)
    inv = np.empty(A, dtype=np.int32)
    n = ctypes.c_int64(0)
    max_tiles = A // tile_m + Ep + 1
    tiles = np.empty((max_tiles, 2), dtype=np.int32)
    check(lib().oracle_align(ptr(flat), A, Ep, tile_m, ptr(counts), ptr(offsets), ptr(srt),
                             ptr(inv), ptr(tiles), max_tiles, ctypes.addressof(n)), "align")
    return counts, offsets, srt, inv, tiles[:n.value].copy(), int(n.value)


def expert_mlp(a: np.ndarray, w13_e, w13s_e, w2_e, w2s_e, I: int, act_fmt: int,
               return_h: bool = False, wfmt: int = W_MXFP4, threads: int | None = None):
    """One expert on rows a (fp64 [n, H], already bf16 / MXFP4-exact values).

    acc = a . dq(W13)^T (fp64); h = bf16(silu(acc[:, :I]) * acc[:, I:]);
    for W4A4 h is MXFP4-quantised along I and decoded; y = h . dq(W2)^T
    (fp64, not rounded).  dq decodes MXFP4 or (wfmt = W_MXFP8) MXFP8
    weights.  With return_h, also returns the bf16 h (before any MXFP4
    step)."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    n, H = a.shape
    arrs = [np.ascontiguousarray(v, dtype=np.uint8) for v in (w13_e, w13s_e, w2_e, w2s_e)]
    y = np.empty((n, H), dtype=np.float64)
    h = np.empty((n, I), dtype=np.float64)
    check(lib().oracle_expert_mlp(ptr(a), n, H, I, *[ptr(v) for v in arrs], act_fmt, wfmt,
                                  ptr(y), ptr(h), threads or default_threads()), "expert_mlp")
    return (y, h) if return_h else y


def quantize_activations(x_bits: np.ndarray):
    """W4A4 activation quantisation: bf16 rows -> MXFP4 (packed, scales)."""
    return mxfp4.quantize(mxfp4.bf16_to_f64(x_bits))


def forward(x_bits, logits, gate, weights, I: int, E: int, K: int, shared: int,
            act_fmt: int = ACT_BF16, tokens=None, renormalize: bool = True,
            tile_m: int = 32, wfmt: int = W_MXFP4, threads: int | None = None,
            return_h: bool = False, round_y: bool = False):
    """The whole layer.

    x_bits uint16 [T, H] (bf16 bit patterns); logits fp32 [T, E]; gate fp32
    [T] or None; weights(e) -> (w13 uint8 [2I, H/2], w13s uint8 [2I, H/32],
    w2 uint8 [H, I/2], w2s uint8 [H, I/32]) for e in [0, E+shared), MXFP4;
    with wfmt = W_MXFP8 the code arrays hold one byte per element (w13
    [2I, H], w2 [H, I]).  MXFP8 weights come with bf16 activations.
    weights(e) is called only for experts the selected tokens use.
    tokens: optional list of token indices; when given, only those tokens'
    outputs are computed (routing and grouping still cover all T tokens).
    return_h (all tokens only): also the bf16 h of every assignment, rows in
    the grouping's sorted order.

    round_y: each slot's expert output y is rounded to bf16 before the
    combine (a path that stores y in bf16 between the down GEMM and the
    combine); False (the default, as the GPU path) keeps it unrounded.
    Returns a dict: ids, w, counts, offsets,
    sorted, inv, tiles, n_tiles, out (uint16 bf16 bits [len(tokens) or T,
    H]), out_f64 (before the last rounding), tokens, seconds (the C++
    call's wall time) and, with return_h, h (uint16 bf16 bits [T*K', I])."""
    assert wfmt == W_MXFP4 or act_fmt == ACT_BF16
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, H = x_bits.shape
    Kp, Ep = K + shared, E + shared
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    g = np.ascontiguousarray(gate, dtype=np.float32) if shared else None
    ids, w = route(logits, g, K, shared, renormalize)
    counts, offsets, srt, inv, tiles, n_tiles = align(ids, Ep, tile_m)
    all_tokens = tokens is None
    tokens = np.arange(T, dtype=np.int64) if all_tokens else np.asarray(tokens, dtype=np.int64)
    assert not (return_h and not all_tokens)
    need = sorted(set(ids[tokens].reshape(-1).tolist())) if len(tokens) else []

    keep = []                                     # the arrays stay alive for the call
    P = ctypes.c_void_p * Ep
    p13, p13s, p2, p2s = P(), P(), P(), P()
    for e in need:
        arrs = [np.ascontiguousarray(v, dtype=np.uint8) for v in weights(int(e))]
        keep.append(arrs)
        for table, arr in zip((p13, p13s, p2, p2s), arrs):
            table[e] = arr.ctypes.data
    n = len(tokens)
    out = np.empty((n, H), dtype=np.uint16)
    out_f64 = np.empty((n, H), dtype=np.float64)
    h = np.empty((T * Kp, I), dtype=np.uint16) if return_h else None
    secs = ctypes.c_double(0.0)
    tok_arg = None if all_tokens else np.ascontiguousarray(tokens)
    check(lib().oracle_forward(ptr(x_bits), ptr(logits), ptr(g), p13, p13s, p2, p2s, T, H, I, E,
                               K, shared, act_fmt, wfmt, int(bool(renormalize)),
                               int(bool(round_y)), ptr(tok_arg),
                               n if not all_tokens else 0, threads or default_threads(), None,
                               None, ptr(out), ptr(out_f64), ptr(h), ctypes.addressof(secs)),
          "forward")
    res = dict(ids=ids, w=w, counts=counts, offsets=offsets, sorted=srt, inv=inv, tiles=tiles,
               n_tiles=n_tiles, out=out, out_f64=out_f64, tokens=tokens, seconds=secs.value)
    if return_h:
        res["h"] = h
    return res


def forward_from_h(h_bits, logits, gate, weights, I: int, E: int, K: int, shared: int,
                   act_fmt: int = ACT_BF16, renormalize: bool = True, wfmt: int = W_MXFP4,
                   threads: int | None = None, round_y: bool = False):
    """The layer from a given h onward: routing and grouping as forward, then
    each assignment's down projection of h_bits (uint16 bf16 [T*K', I], rows
    in the grouping's sorted order; MXFP4-quantised and decoded first for
    W4A4) and the combine.  weights(e) as in forward (only its W2 arrays
    are read).  Returns out (bf16 bits [T, H]) and out_f64."""
    h_bits = np.ascontiguousarray(h_bits, dtype=np.uint16)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T = logits.shape[0]
    Kp, Ep = K + shared, E + shared
    assert h_bits.shape == (T * Kp, I)
    g = np.ascontiguousarray(gate, dtype=np.float32) if shared else None
    ids, _ = route(logits, g, K, shared, renormalize)
    keep = []
    P = ctypes.c_void_p * Ep
    p2, p2s = P(), P()
    for e in sorted(set(ids.reshape(-1).tolist())):
        arrs = [np.ascontiguousarray(v, dtype=np.uint8) for v in weights(int(e))[2:4]]
        keep.append(arrs)
        p2[e], p2s[e] = arrs[0].ctypes.data, arrs[1].ctypes.data
    H = keep[0][0].shape[0] if keep else 0
    out = np.empty((T, H), dtype=np.uint16)
    out_f64 = np.empty((T, H), dtype=np.float64)
    check(lib().oracle_forward_from_h(ptr(h_bits), ptr(logits), ptr(g), p2, p2s, T, H, I, E, K,
                                      shared, act_fmt, wfmt, int(bool(renormalize)),
                                      int(bool(round_y)), threads or default_threads(), ptr(out),
                                      ptr(out_f64)), "forward_from_h")
    return dict(out=out, out_f64=out_f64)


def weights_from_arrays(w13, w13s, w2, w2s):
    """Adapter: stacked arrays [E', ...] -> the weights(e) callable."""
    return lambda e: (w13[e], w13s[e], w2[e], w2s[e])
