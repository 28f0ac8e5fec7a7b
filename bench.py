"""Throughput of the MXFP4 routed-expert MoE layer on one MI355X.

One step = one pass of the whole layer (route, align, [quantise x], gate/up
+ SwiGLU, [quantise h], down, combine) over one batch, through the C ABI, on
inputs already resident in HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

The default workload is the decode batch (T=64, H=4096, I=1024, E=512,
top-10 + shared expert, W4A16).  The cpu_baseline leg times the CPU oracle
on a few tokens of the same batch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

import synth

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
MXFP4_PEAK_TFLOPS = 10100.0      # dense MXFP4 MFMA
BF16_PEAK_TFLOPS = 2500.0        # dense bf16 MFMA
METRIC = "MoE-layer tokens/s; % HBM peak (decode T=64), % MXFP4 MFMA peak (prefill)"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode", choices=list(synth.CONFIGS))
    p.add_argument("--cpu-tokens", type=int, default=3,
                   help="tokens of the batch the CPU oracle is timed on")
    p.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_inputs(cfg):
    from mxfp4_routed_expert_top_amd import ops
    dev = "cuda"
    x = synth.activations(cfg).to(dev)
    logits = synth.router_logits(cfg).to(dev)
    gate = synth.gate_logits(cfg)
    gate = None if gate is None else gate.to(dev)
    u8 = dict(dtype=torch.uint8, device=dev)
    w13 = torch.empty(cfg.Ep, 2 * cfg.I, cfg.H // 2, **u8)
    w13s = torch.empty(cfg.Ep, 2 * cfg.I, cfg.H // 32, **u8)
    w2 = torch.empty(cfg.Ep, cfg.H, cfg.I // 2, **u8)
    w2s = torch.empty(cfg.Ep, cfg.H, cfg.I // 32, **u8)
    for e in range(cfg.Ep):             # float draws packed by the library's own quantiser
        ops.mxfp4_quantize(synth.expert_w13(cfg, e, dev), w13[e], w13s[e])
        ops.mxfp4_quantize(synth.expert_w2(cfg, e, dev), w2[e], w2s[e])
    torch.cuda.synchronize()
    return x, logits, gate, w13, w13s, w2, w2s


def algorithmic(cfg, counts):
    """Bytes the layer must move and FLOPs it must do, given the realised
    per-expert counts (weights of experts that got no token are not counted)."""
    touched = int((counts > 0).sum())
    w13_e = 2 * cfg.I * cfg.H // 2 + 2 * cfg.I * cfg.H // 32
    w2_e = cfg.H * cfg.I // 2 + cfg.H * cfg.I // 32
    io = cfg.T * cfg.H * 2 + cfg.T * cfg.E * 4 + cfg.T * 4 * cfg.shared + cfg.T * cfg.H * 2
    return dict(touched=touched, w13_bytes=touched * w13_e, w2_bytes=touched * w2_e,
                layer_bytes=touched * (w13_e + w2_e) + io,
                flops=cfg.A * 6 * cfg.H * cfg.I, gate_up_flops=cfg.A * 4 * cfg.H * cfg.I)


def cpu_baseline(cfg, w13_dev_fn, n_tokens):
    """Time the oracle (as it stands) on n_tokens of the batch."""
    from oracle import moe, mxfp4
    from threadpoolctl import threadpool_info
    x_bits = synth.activations(cfg).view(torch.int16).numpy().view(np.uint16)
    logits = synth.router_logits(cfg).numpy()
    gate = synth.gate_logits(cfg)
    gate = None if gate is None else gate.numpy()
    tokens = np.arange(n_tokens)
    ids, _ = moe.route(logits, gate, cfg.K, cfg.shared)
    need = sorted(set(ids[tokens].reshape(-1).tolist()))
    log(f"cpu_baseline: packing {len(need)} experts with the oracle's quantiser")
    packed = {}
    for e in need:
        a = mxfp4.quantize(synth.expert_w13(cfg, e, "cuda").cpu().double().numpy())
        b = mxfp4.quantize(synth.expert_w2(cfg, e, "cuda").cpu().double().numpy())
        packed[e] = (a[0], a[1], b[0], b[1])
    t0 = time.perf_counter()
    moe.forward(x_bits, logits, gate, lambda e: packed[e], cfg.I, cfg.E, cfg.K, cfg.shared,
                cfg.act_fmt, tokens=tokens)
    dt = time.perf_counter() - t0
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": max(blas + [1]),
            "kind": "oracle", "seconds": dt,
            "sample": f"first {n_tokens} of the {cfg.T} tokens ({len(need)} experts), "
                      "routing and grouping over all tokens; numpy fp64, BLAS threads = cores"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(this layer is measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    from mxfp4_routed_expert_top_amd import ops
    cfg = synth.CONFIGS[args.workload]
    log(f"workload {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} K={cfg.K} "
        f"shared={cfg.shared} act={'mxfp4' if cfg.act_fmt else 'bf16'}")
    x, logits, gate, w13, w13s, w2, w2s = make_inputs(cfg)
    bufs = ops.alloc_stages(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, cfg.shared, cfg.act_fmt, "cuda")
    names = ["route", "align", "gate_up", "down", "combine"]
    if cfg.act_fmt == ops.ACT_MXFP4:
        names += ["quant_x", "quant_h"]

    def step(events=None):
        ops.forward_stages(x, logits, gate, w13, w13s, w2, w2s, cfg.I, cfg.E, cfg.K, cfg.shared,
                           cfg.act_fmt, bufs=bufs, events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    ev = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for n in names} for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    stage_ms = {n: float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in ev])) for n in names}
    log("stage ms:", json.dumps({k: round(v, 4) for k, v in stage_ms.items()}))

    counts = bufs["align"]["counts"].cpu().numpy()
    alg = algorithmic(cfg, counts)
    gu_s = stage_ms["gate_up"] / 1e3
    achieved = alg["w13_bytes"] / gu_s / 1e9
    layer_s = ms / 1e3
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "gate_up_w4a16_kernel" if cfg.act_fmt == 0 else "gate_up_w4a4_kernel",
                "algorithmic_bytes": alg["w13_bytes"], "kernel_ms": round(stage_ms["gate_up"], 4)}
    layer = {"bytes": alg["layer_bytes"], "flops": alg["flops"], "touched_experts": alg["touched"],
             "hbm_frac": round(alg["layer_bytes"] / layer_s / 1e9 / HBM_PEAK_GBS, 4),
             "mxfp4_mfma_frac": round(alg["flops"] / layer_s / 1e12 / MXFP4_PEAK_TFLOPS, 5),
             "bf16_mfma_frac": round(alg["flops"] / layer_s / 1e12 / BF16_PEAK_TFLOPS, 5),
             "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()}}
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, None, args.cpu_tokens)
    res = {"metric": METRIC, "value": round(cfg.T / layer_s, 1), "unit": "tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if cfg.act_fmt == 0 else "mxfp4",
           "data": "synthetic",
           "config": {"workload": f"{cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} "
                                  f"K={cfg.K}+{cfg.shared} shared, "
                                  f"{'W4A16' if cfg.act_fmt == 0 else 'W4A4'} MXFP4 weights",
                      "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "K": cfg.K,
                      "shared": cfg.shared, "parallelism": "none (1 GPU)"},
           "roofline": roofline, "layer": layer, "cpu_baseline": cpu}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
