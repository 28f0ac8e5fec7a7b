"""Seeded synthetic inputs for the MXFP4 routed-expert MoE layer.

This module is shared by the HIP path's tests and bench and by the CPU
oracle.  It holds random draws and nothing else: no routing, no MXFP4
encoding, no GEMM, no rounding rule of the method.  Weights are produced
here as float32 draws; each side packs them to MXFP4 with its own
quantiser (the oracle with ``oracle.mxfp4.quantize``, the GPU path with
``moe_mxfp4_quantize``), and the two packings are compared bit for bit.

Shapes follow the workloads the pages describe:

* 512 routed MXFP4 experts with softmax top-10 routing and the shared
  expert folded in as one more expert (InferenceX "MI355X Qwen3.5 SGLang
  v0.5.12" post, section on the specific optimisations: the shared-expert
  fusion and fused_topk bullets; VibeSys "Qwen3.5-397B on 4x MI300A" post,
  section "Goal").
* a decode batch of 64 tokens, a packed 1,536-token prefill chunk (VibeSys
  post, section "Prefill, cache and speculation") and an 8,192-token
  prefill chunk (OpenRelay "Gemma 4 31B on MI355X" post, section
  "Optimisation 4").

Every draw comes from ``torch.Generator`` seeded by a fixed integer derived
from (config seed, stream id, index).  Activations, router logits and gate
logits are always drawn on the CPU so that every machine sees the same
values; expert weights may be drawn on the GPU for the full-size shapes
(drawing 6.4e9 normals on the host would take minutes), and then the same
tensor is copied to the host for the oracle.
"""
from __future__ import annotations

import math
import dataclasses
from dataclasses import dataclass, field

import torch

# stream ids: one per kind of draw
STREAM_X = 1
STREAM_LOGITS = 2
STREAM_GATE = 3
STREAM_W13 = 4
STREAM_W2 = 5
STREAM_OUTLIER = 6
STREAM_SKEW = 7
STREAM_ROUTER = 8
STREAM_NORM = 9

ACT_BF16 = 0    # W4A16: bf16 activations
ACT_MXFP4 = 1   # W4A4: activations quantised to MXFP4 on the fly

# Popularity exponent of the skewed router bias and the fraction of
# assignments its top 5% of experts should take (40 +- 1 %).  SKEW_BETA was
# found by bisection with oracle/calibrate_skew.py on the draw of the
# "prefill_skewed" workload below; tests/test_synth.py re-checks the share.
ZIPF_S = 1.1
SKEW_BETA = 0.3848


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                 # tokens
    H: int                 # hidden size
    I: int                 # expert intermediate size
    E: int                 # routed experts
    K: int                 # routed top-K
    shared: int            # 1: shared expert folded in as expert E, slot K
    act_fmt: int           # ACT_BF16 or ACT_MXFP4
    seed_act: int          # seed of x, logits, gate
    seed_w: int            # seed of the expert weights
    w_std: float = 0.02
    skew: bool = False     # Zipf-biased router logits with 3 dead experts
    outlier_p: float = 0.0 # fraction of activations multiplied by outlier_mult
    outlier_mult: float = 50.0
    wfmt: int = 0          # expert weights packed as W_MXFP4 or W_MXFP8

    @property
    def Kp(self) -> int:
        return self.K + self.shared

    @property
    def Ep(self) -> int:
        return self.E + self.shared

    @property
    def A(self) -> int:
        return self.T * self.Kp


W_MXFP4, W_MXFP8 = 0, 1

# The workloads.  "decode" is the one the throughput line is quoted on;
# "decode_mxfp8" is the same batch and the same weight draws packed as MXFP8.
CONFIGS = {
    "tiny": MoEConfig("tiny", T=8, H=256, I=128, E=16, K=2, shared=0,
                      act_fmt=ACT_BF16, seed_act=1000, seed_w=70),
    "decode": MoEConfig("decode", T=64, H=4096, I=1024, E=512, K=10, shared=1,
                        act_fmt=ACT_BF16, seed_act=1001, seed_w=77),
    "prefill": MoEConfig("prefill", T=1536, H=4096, I=1024, E=512, K=10, shared=1,
                         act_fmt=ACT_BF16, seed_act=1002, seed_w=77),
    "prefill_skewed": MoEConfig("prefill_skewed", T=8192, H=4096, I=1024, E=512, K=10,
                                shared=1, act_fmt=ACT_BF16, seed_act=1003, seed_w=77,
                                skew=True),
    "w4a4": MoEConfig("w4a4", T=4096, H=6144, I=1536, E=256, K=8, shared=1,
                      act_fmt=ACT_MXFP4, seed_act=1004, seed_w=74, outlier_p=0.001),
    "decode_mxfp8": MoEConfig("decode_mxfp8", T=64, H=4096, I=1024, E=512, K=10, shared=1,
                              act_fmt=ACT_BF16, seed_act=1001, seed_w=77, wfmt=W_MXFP8),
    "prefill_mxfp8": MoEConfig("prefill_mxfp8", T=1536, H=4096, I=1024, E=512, K=10, shared=1,
                               act_fmt=ACT_BF16, seed_act=1002, seed_w=77, wfmt=W_MXFP8),
    # one GPU's share of the decode layer split 8 ways by tensor parallelism:
    # every expert's I/8 slice of gate/up rows and down columns
    "decode_tp8": MoEConfig("decode_tp8", T=64, H=4096, I=128, E=512, K=10, shared=1,
                            act_fmt=ACT_BF16, seed_act=1001, seed_w=77),
}


def layer_config(cfg: MoEConfig, layer: int) -> MoEConfig:
    """The config of layer `layer` of a multi-layer pass: the same shapes with
    its own weight and router-row draws (layer 0 is cfg itself)."""
    if layer == 0:
        return cfg
    return dataclasses.replace(cfg, name=f"{cfg.name}_layer{layer}",
                               seed_w=cfg.seed_w + 1000 * layer, seed_act=cfg.seed_act + 1000 * layer)


def custom_config(name="custom", **kw) -> MoEConfig:
    """A config of any shape for tests (defaults: small W4A16 with shared)."""
    base = dict(T=40, H=256, I=128, E=16, K=4, shared=1, act_fmt=ACT_BF16,
                seed_act=7, seed_w=8)
    base.update(kw)
    return MoEConfig(name, **base)


def _seed(seed: int, stream: int, index: int = 0) -> int:
    # a fixed injective-enough mix of the three integers into a 63-bit seed
    return (seed * 1_000_003 + stream * 10_007 + index * 97 + 12345) % (2**63 - 1)


def _gen(seed: int, stream: int, index: int = 0, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, stream, index))
    return g


def activations(cfg: MoEConfig) -> torch.Tensor:
    """x: bf16 [T, H], N(0,1), with a Bernoulli(outlier_p) mask scaled by
    outlier_mult before the cast to bf16 (CPU tensor)."""
    x = torch.randn(cfg.T, cfg.H, generator=_gen(cfg.seed_act, STREAM_X), dtype=torch.float32)
    if cfg.outlier_p > 0:
        u = torch.rand(cfg.T, cfg.H, generator=_gen(cfg.seed_act, STREAM_OUTLIER))
        x = torch.where(u < cfg.outlier_p, x * cfg.outlier_mult, x)
    return x.to(torch.bfloat16)


def skew_bias(cfg: MoEConfig, beta: float = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Per-expert router bias b_e = -beta * s * ln(rank_e) with Zipf exponent
    s; ranks come from a seeded permutation.  Three experts of rank above the
    top 5% get a bias of -1e4, so they are never selected.
    Returns (bias fp32 [E], dead expert ids int64 [3])."""
    beta = SKEW_BETA if beta is None else beta
    g = _gen(cfg.seed_act, STREAM_SKEW)
    perm = torch.randperm(cfg.E, generator=g)            # perm[r] = expert of rank r+1
    rank = torch.empty(cfg.E, dtype=torch.float64)
    rank[perm] = torch.arange(1, cfg.E + 1, dtype=torch.float64)
    bias = -beta * ZIPF_S * torch.log(rank)
    n_top = math.ceil(0.05 * cfg.E)
    tail = perm[n_top:]
    pick = torch.randperm(tail.numel(), generator=g)[:3]
    dead = torch.sort(tail[pick]).values
    bias[dead] = -1.0e4
    return bias.to(torch.float32), dead


def router_logits(cfg: MoEConfig, beta: float = None) -> torch.Tensor:
    """logits: fp32 [T, E], N(0,1) (+ skew bias for the skewed workload)."""
    l = torch.randn(cfg.T, cfg.E, generator=_gen(cfg.seed_act, STREAM_LOGITS), dtype=torch.float32)
    if cfg.skew:
        bias, _ = skew_bias(cfg, beta)
        l = l + bias[None, :]
    return l


def gate_logits(cfg: MoEConfig):
    """Shared-expert gate logits g: fp32 [T], N(0,1); None without a shared expert."""
    if not cfg.shared:
        return None
    return torch.randn(cfg.T, generator=_gen(cfg.seed_act, STREAM_GATE), dtype=torch.float32)


def expert_w13(cfg: MoEConfig, e: int, device="cpu") -> torch.Tensor:
    """Gate/up weights of expert e: fp32 [2I, H] ~ N(0, w_std); rows [0, I)
    are the gate projection, rows [I, 2I) the up projection."""
    g = _gen(cfg.seed_w, STREAM_W13, e, device)
    return torch.randn(2 * cfg.I, cfg.H, generator=g, device=device, dtype=torch.float32).mul_(cfg.w_std)


def expert_w2(cfg: MoEConfig, e: int, device="cpu") -> torch.Tensor:
    """Down weights of expert e: fp32 [H, I] ~ N(0, w_std)."""
    g = _gen(cfg.seed_w, STREAM_W2, e, device)
    return torch.randn(cfg.H, cfg.I, generator=g, device=device, dtype=torch.float32).mul_(cfg.w_std)


def router_weight(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    """Router rows for the router GEMM: bf16 [E + shared, H] ~ N(0, 1/H), so
    that x . Wr^T has roughly unit variance like the drawn logits; row E
    (with a shared expert) is the shared expert's gate vector."""
    g = _gen(cfg.seed_act, STREAM_ROUTER, 0, device)
    w = torch.randn(cfg.E + cfg.shared, cfg.H, generator=g, device=device, dtype=torch.float32)
    return w.mul_(cfg.H ** -0.5).to(torch.bfloat16)


def ties_logits(T: int, E: int, seed: int) -> torch.Tensor:
    """Router logits full of exact ties and signed zeros: values drawn from
    {-0.0, +0.0, +-0.5, +-1.0} so that top-K must break ties by index."""
    g = _gen(seed, STREAM_LOGITS, 99)
    vals = torch.tensor([-0.0, 0.0, 0.5, -0.5, 1.0, -1.0], dtype=torch.float32)
    idx = torch.randint(0, vals.numel(), (T, E), generator=g)
    return vals[idx]


def norm_inputs(G: int, T: int, H: int, seed: int, part_std: float = 0.5):
    """Inputs of the step after the layer (partial outputs summed, residual
    added, RMSNorm): G partial outputs bf16 [G, T, H] ~ N(0, part_std^2)
    (one tensor-parallel rank's share of the layer output each), the residual
    stream bf16 [T, H] ~ N(0, 1) and gamma bf16 [H] ~ U(0.5, 1.5)
    (CPU tensors)."""
    g = _gen(seed, STREAM_NORM)
    p = torch.randn(G, T, H, generator=g, dtype=torch.float32).mul_(part_std)
    r = torch.randn(T, H, generator=g, dtype=torch.float32)
    gamma = torch.rand(H, generator=g, dtype=torch.float32).add_(0.5)
    return p.to(torch.bfloat16), r.to(torch.bfloat16), gamma.to(torch.bfloat16)
