"""The MXFP4 routed-expert MoE layer, computed from its plain definition (fp64).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package.  It shares no code with the HIP
path and never imports it.

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
  out_t = bf16( sum_k w_t,k * bf16(MLP_{e_k}(x_t)) ), summed in slot order.

MXFP4 weights are decoded exactly; each dot product is an fp64 matmul over
exact products; bf16 rounding happens where the GPU path stores bf16: h,
each slot's expert output y (staged between the down GEMM and the combine;
the pages fix no precision for it, and bf16 is the activations' type on the
path) and out.  For W4A4 the activations and h are MXFP4-quantised then decoded
before their GEMM (OpenRelay "Gemma 4 31B on MI355X" post, sections
"Optimisation 3" and "Optimisation 4": activation + MXFP4 quantisation
fused into one kernel).

Grouping by expert (align) is defined here as a stable sort of the flat
assignment ids t*K'+k by expert id; the tile list is the 32-row tiles of
each expert's group (VibeSys post, section "Prefill, cache and
speculation": 32-row tiles in the MoE kernel).

The router GEMM that produces the logits (the step before routing; the
InferenceX post's fused_topk consumes a separately computed gating output)
is logits = x . Wr^T over bf16 x and bf16 router rows, and with a shared
expert the gate logit g = x . Wr[E] of one more row: router_logits computes
it exactly (fp64 sums of exact products).

Expert weights may also be MXFP8 (oracle/mxfp8.py), with bf16 activations;
everything else is unchanged.

Pins: tests/test_oracle_moe.py, tests/golden/route_align.json.
"""
from __future__ import annotations

import numpy as np

from . import mxfp4, mxfp8

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
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = l.shape
    Kp = K + shared
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -l), axis=-1)[:, :K]       # primary key -l, then index
    ids = np.empty((T, Kp), dtype=np.int32)
    w = np.empty((T, Kp), dtype=np.float32)
    ids[:, :K] = order
    top = np.take_along_axis(l, order, axis=1)
    lmax = l.max(axis=1, keepdims=True)
    num = np.exp(top - lmax)
    den = num.sum(axis=1, keepdims=True) if renormalize else np.exp(l - lmax).sum(axis=1, keepdims=True)
    w[:, :K] = (num / den).astype(np.float32)
    if shared:
        g = np.asarray(gate, dtype=np.float32).astype(np.float64)
        ids[:, K] = E
        w[:, K] = (1.0 / (1.0 + np.exp(-g))).astype(np.float32)
    return ids, w


def router_logits(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """Router GEMM: x bf16 bits [T, H], router rows bf16 bits [R, H] ->
    fp64 [T, R] = x . W^T.  The inputs are decoded exactly and each product
    of two bf16 values is exact in fp64; the sums are fp64 (exact unless a
    row's products span more than fp64's 53 bits of magnitude)."""
    x = mxfp4.bf16_to_f64(x_bits)
    w = mxfp4.bf16_to_f64(w_bits)
    return x @ w.T


def align(ids: np.ndarray, Ep: int, tile_m: int = 32):
    """Group the flat assignments a = t*K'+k by expert, stably.

    Returns counts int32 [Ep], offsets int32 [Ep+1] (exclusive scan, the
    last entry = A), sorted int32 [A] (flat ids grouped by expert,
    ascending inside a group), inv int32 [A] (position of each flat id in
    sorted), tiles int32 [n_tiles, 2] (expert, first row) for tile_m-row
    tiles, expert-major and ascending, and n_tiles."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    A = flat.size
    counts = np.bincount(flat, minlength=Ep)[:Ep].astype(np.int32)
    offsets = np.zeros(Ep + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_ = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty(A, dtype=np.int32)
    inv[sorted_] = np.arange(A, dtype=np.int32)
    tiles = [(e, offsets[e] + s) for e in range(Ep) for s in range(0, int(counts[e]), tile_m)]
    tiles = np.array(tiles, dtype=np.int32).reshape(-1, 2)
    return counts, offsets, sorted_, inv, tiles, len(tiles)


def silu(z):
    """z * sigmoid(z) in fp64."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_mlp(a: np.ndarray, w13_e, w13s_e, w2_e, w2s_e, I: int, act_fmt: int,
               return_h: bool = False, wfmt: int = W_MXFP4):
    """One expert on rows a (fp64 [n, H], already bf16 / MXFP4-exact values).

    acc = a . dq(W13)^T (fp64); h = bf16(silu(acc[:, :I]) * acc[:, I:]);
    for W4A4 h is MXFP4-quantised along I and decoded; y = h . dq(W2)^T.
    dq decodes MXFP4 or (wfmt = W_MXFP8) MXFP8 weights.  With return_h, also
    returns the bf16 h (before any MXFP4 step)."""
    W13 = decode_weights(w13_e, w13s_e, wfmt)      # [2I, H]
    acc = a @ W13.T                                # [n, 2I]
    h = mxfp4.round_bf16(silu(acc[:, :I]) * acc[:, I:])
    hin = mxfp4.decode(*mxfp4.quantize(h)) if act_fmt == ACT_MXFP4 else h
    W2 = decode_weights(w2_e, w2s_e, wfmt)         # [H, I]
    y = hin @ W2.T                                 # [n, H]
    return (y, h) if return_h else y


def quantize_activations(x_bits: np.ndarray):
    """W4A4 activation quantisation: bf16 rows -> MXFP4 (packed, scales)."""
    return mxfp4.quantize(mxfp4.bf16_to_f64(x_bits))


def forward(x_bits, logits, gate, weights, I: int, E: int, K: int, shared: int,
            act_fmt: int = ACT_BF16, tokens=None, renormalize: bool = True,
            tile_m: int = 32, wfmt: int = W_MXFP4):
    """The whole layer.

    x_bits uint16 [T, H] (bf16 bit patterns); logits fp32 [T, E]; gate fp32
    [T] or None; weights(e) -> (w13 uint8 [2I, H/2], w13s uint8 [2I, H/32],
    w2 uint8 [H, I/2], w2s uint8 [H, I/32]) for e in [0, E+shared), MXFP4;
    with wfmt = W_MXFP8 the code arrays hold one byte per element (w13
    [2I, H], w2 [H, I]).  MXFP8 weights come with bf16 activations.
    tokens: optional list of token indices; when given, only those tokens'
    outputs are computed (routing and grouping still cover all T tokens).

    Each slot's expert output y is rounded to bf16 before the combine (where
    the GPU path stores it).  Returns a dict: ids, w, counts, offsets,
    sorted, inv, tiles, n_tiles, out (uint16 bf16 bits [len(tokens) or T,
    H]), out_f64 (before the last rounding), tokens."""
    assert wfmt == W_MXFP4 or act_fmt == ACT_BF16
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, H = x_bits.shape
    Kp, Ep = K + shared, E + shared
    ids, w = route(logits, gate, K, shared, renormalize)
    counts, offsets, sorted_, inv, tiles, n_tiles = align(ids, Ep, tile_m)
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)

    if act_fmt == ACT_MXFP4:
        xq, xs = quantize_activations(x_bits[tokens])
        a_all = mxfp4.decode(xq, xs)
    else:
        a_all = mxfp4.bf16_to_f64(x_bits[tokens])

    # y[j, k] = MLP of slot k of token tokens[j]
    y = np.zeros((len(tokens), Kp, H), dtype=np.float64)
    sel_ids = ids[tokens]                          # [n, Kp]
    for e in np.unique(sel_ids):
        rows, slots = np.nonzero(sel_ids == e)
        y[rows, slots] = mxfp4.round_bf16(expert_mlp(a_all[rows], *weights(int(e)), I, act_fmt,
                                                     wfmt=wfmt))

    acc = np.zeros((len(tokens), H), dtype=np.float64)
    wt = w[tokens].astype(np.float64)
    for k in range(Kp):                            # slot order
        acc += wt[:, k, None] * y[:, k]
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, sorted=sorted_, inv=inv,
                tiles=tiles, n_tiles=n_tiles, out=mxfp4.bf16_bits(acc), out_f64=acc,
                tokens=tokens)


def weights_from_arrays(w13, w13s, w2, w2s):
    """Adapter: stacked arrays [E', ...] -> the weights(e) callable."""
    return lambda e: (w13[e], w13s[e], w2[e], w2s[e])
