"""Throughput of the MXFP4 routed-expert MoE layer on one MI355X.

One step = one pass of the whole layer (route, align, [quantise x], gate/up
+ SwiGLU, [quantise h], down, combine) over one batch, through the C ABI, on
inputs already resident in HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

The default workload is the decode batch (T=64, H=4096, I=1024, E=512,
top-10 + shared expert, W4A16); its throughput is `value`.  The same run
also times the prefill chunk (T=1536), the skewed prefill chunk (T=8192)
and the W4A4 batch (T=4096, H=6144, I=1536, E=256, top-8 + shared) and
reports each under `workloads` with its rooflines.  The cpu_baseline leg
times the C++ CPU oracle on the whole decode batch on the host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
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
    p.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    p.add_argument("--no-extras", action="store_true",
                   help="time only the decode workload (by default the prefill, skewed prefill "
                        "and W4A4 workloads are timed too, under 'workloads')")
    p.add_argument("--no-sha", dest="sha", action="store_false",
                   help="skip the SHA-256 of the input buffers")
    p.add_argument("--router", action="store_true",
                   help="route from x through the router GEMM (bf16 router rows [E + shared, H]) "
                        "instead of taking precomputed logits")
    p.add_argument("--layers", type=int, default=0,
                   help="time L layers of the workload (each its own weights and router rows) "
                        "in one moe_mxfp4_forward_layers call, eager and replayed from a HIP graph")
    p.add_argument("--norm", action="store_true",
                   help="with --layers: the residual add and RMSNorm after each layer "
                        "(moe_mxfp4_forward_layers_norm)")
    p.add_argument("--prefetch", action="store_true",
                   help="with --layers: each layer's combine prefetches the next layer's router "
                        "rows and shared expert into the caches")
    p.add_argument("--epilogue", type=int, nargs="*", default=None, metavar="T",
                   help="time only the step after the layer at tensor-parallel degree 8 "
                        "(partials summed, residual added, RMSNorm) for these batch sizes "
                        "(default: 64, 1536 and 8192 tokens) and print its record")
    p.add_argument("--pmc-calibrate", action="store_true",
                   help="first run a plain 1 GiB kernel (torch.bitwise_not) whose HBM bytes are "
                        "known, for scaling FETCH_SIZE / WRITE_SIZE counter passes")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_inputs(cfg, weights=None):
    """x, logits, gate of the workload on the GPU, and its expert weights
    (drawn and packed by the library's quantiser unless `weights` holds the
    same draw's packing already)."""
    from mxfp4_routed_expert_top_amd import ops
    dev = "cuda"
    x = synth.activations(cfg).to(dev)
    logits = synth.router_logits(cfg).to(dev)
    gate = synth.gate_logits(cfg)
    gate = None if gate is None else gate.to(dev)
    if weights is not None:
        return (x, logits, gate, *weights)
    u8 = dict(dtype=torch.uint8, device=dev)
    per = 1 if cfg.wfmt == synth.W_MXFP8 else 2      # elements per code byte
    w13 = torch.empty(cfg.Ep, 2 * cfg.I, cfg.H // per, **u8)
    w13s = torch.empty(cfg.Ep, 2 * cfg.I, cfg.H // 32, **u8)
    w2 = torch.empty(cfg.Ep, cfg.H, cfg.I // per, **u8)
    w2s = torch.empty(cfg.Ep, cfg.H, cfg.I // 32, **u8)
    for e in range(cfg.Ep):             # float draws packed by the library's own quantiser
        ops.quantize_weights(synth.expert_w13(cfg, e, dev), w13[e], w13s[e], cfg.wfmt)
        ops.quantize_weights(synth.expert_w2(cfg, e, dev), w2[e], w2s[e], cfg.wfmt)
    torch.cuda.synchronize()
    return x, logits, gate, w13, w13s, w2, w2s


def algorithmic(cfg, counts):
    """Bytes the layer must move and FLOPs it must do, given the realised
    per-expert counts (weights of experts that got no token are not counted;
    intermediates such as h and y are implementation traffic, not counted).
    gate_up's own figure: the touched experts' W13 codes + scales and the
    activations it reads (bf16 x, or its MXFP4 codes + scales for W4A4)."""
    touched = int((counts > 0).sum())
    per = 1 if cfg.wfmt == synth.W_MXFP8 else 2      # elements per code byte
    w13_e = 2 * cfg.I * cfg.H // per + 2 * cfg.I * cfg.H // 32
    w2_e = cfg.H * cfg.I // per + cfg.H * cfg.I // 32
    io = cfg.T * cfg.H * 2 + cfg.T * cfg.E * 4 + cfg.T * 4 * cfg.shared + cfg.T * cfg.H * 2
    x_gu = cfg.T * cfg.H * 2 if cfg.act_fmt == 0 else cfg.T * (cfg.H // 2 + cfg.H // 32)
    return dict(touched=touched, w13_bytes=touched * w13_e, w2_bytes=touched * w2_e,
                gate_up_bytes=touched * w13_e + x_gu,
                layer_bytes=touched * (w13_e + w2_e) + io,
                flops=cfg.A * 6 * cfg.H * cfg.I, gate_up_flops=cfg.A * 4 * cfg.H * cfg.I)


def gate_up_kernel_name(cfg, tile_m):
    """The gate/up kernel's name as rocprofv3 reports it for this shape."""
    a = "true" if cfg.act_fmt else "false"
    w8 = "true" if cfg.wfmt == synth.W_MXFP8 else "false"
    if tile_m != 32:
        # variants of the MXFP4-activation 128-row kernel by reduction length
        kv = 0
        if cfg.act_fmt and tile_m == 128:
            kv = 1 if cfg.H <= 2048 else 2 if cfg.H <= 6144 else 0
        # the forward feeds MXFP4 activations to the tiled kernels in the blocked row order
        # and then quantises h in the gate/up epilogue
        blk = "true" if cfg.act_fmt else "false"
        return f"gate_up_tiled_kernel<{tile_m}, {a}, {w8}, {kv}, {blk}, {blk}>"
    if cfg.wfmt == synth.W_MXFP8:
        return "gate_up_kernel<1, false, true>"
    ph = 2 if (cfg.H // 128) % 2 == 0 else 1          # phase width of the 32-row kernel
    return f"gate_up_kernel<{ph}, {a}, false>"


def traffic_path(cfg):
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"{cfg.name}_T{cfg.T}_traffic.json")


def sha256_of(*tensors: torch.Tensor) -> str:
    """SHA-256 of the tensors' bytes, one after another (copied to the host
    in slices)."""
    h = hashlib.sha256()
    step = 64 << 20
    for t in tensors:
        flat = t.detach().contiguous().view(-1).view(torch.uint8)
        for lo in range(0, flat.numel(), step):
            h.update(flat[lo:lo + step].cpu().numpy().tobytes())
    return h.hexdigest()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(cfg, router=False):
    """Time the C++ oracle, as it stands, on the whole batch: routing and
    grouping of every token, every touched expert's MLP in fp64, the
    combine (oracle_forward's own wall time).  Threads: the CPUs of the
    affinity mask (at most 16, one GPU's share of the host).  Its weights are
    the same float draws (drawn on the GPU by the seeded generator, copied to
    the host) packed by the oracle's own quantiser beforehand (not timed)."""
    from oracle import _lib as olib
    from oracle import moe, mxfp4, mxfp8
    threads = olib.default_threads()
    x_bits = synth.activations(cfg).view(torch.int16).numpy().view(np.uint16)
    t_router = 0.0
    if router:
        wr_bits = synth.router_weight(cfg).view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        lg = moe.router_logits(x_bits, wr_bits, threads=threads)
        t_router = time.perf_counter() - t0
        logits = lg[:, :cfg.E].astype(np.float32)
        gate = lg[:, cfg.E].astype(np.float32) if cfg.shared else None
    else:
        logits = synth.router_logits(cfg).numpy()
        gate = synth.gate_logits(cfg)
        gate = None if gate is None else gate.numpy()
    ids, _ = moe.route(logits, gate, cfg.K, cfg.shared)
    need = sorted(set(ids.reshape(-1).tolist()))
    q = mxfp8.quantize if cfg.wfmt == synth.W_MXFP8 else mxfp4.quantize
    log(f"cpu_baseline: packing {len(need)} experts with the oracle's quantiser ({threads} threads)")
    packed = {}
    for e in need:
        a = q(synth.expert_w13(cfg, e, "cuda").cpu().numpy(), threads=threads)
        b = q(synth.expert_w2(cfg, e, "cuda").cpu().numpy(), threads=threads)
        packed[e] = (a[0], a[1], b[0], b[1])
    log("cpu_baseline: timing oracle_forward on the whole batch")
    res = moe.forward(x_bits, logits, gate, lambda e: packed[e], cfg.I, cfg.E, cfg.K, cfg.shared,
                      cfg.act_fmt, wfmt=cfg.wfmt, threads=threads)
    dt = res["seconds"] + t_router
    flops = cfg.A * 6 * cfg.H * cfg.I + (2 * cfg.T * cfg.Ep * cfg.H if router else 0)
    return {"value": round(cfg.T / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3), "gflops_fp64": round(flops / dt / 1e9, 2),
            "cpu": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"the whole batch: {cfg.T} tokens, {cfg.A} assignments, {len(need)} experts "
                      "decoded" + (", router GEMM included" if router else "")
                      + "; C++ fp64 oracle (oracle_forward), one std::thread pool"}


def bench_layers(cfg, args):
    """--layers L: the MoE part of a decode step through L layers in one C call
    (router GEMM + the layer, per layer), eager and as one HIP graph."""
    from mxfp4_routed_expert_top_amd import ops
    L, dev = args.layers, "cuda"
    x = synth.activations(cfg).to(dev)
    layers = []
    for l in range(L):
        lc = synth.layer_config(cfg, l)
        _, _, _, w13, w13s, w2, w2s = make_inputs(lc)
        layers.append((synth.router_weight(lc).to(dev), w13, w13s, w2, w2s))
        log(f"layer {l} weights ready")
    ws = torch.empty(ops.workspace_size(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, cfg.shared, cfg.act_fmt),
                     dtype=torch.uint8, device=dev)
    out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device=dev)
    pf = 1 if args.prefetch else 0
    s = torch.cuda.Stream()
    norm = bool(args.norm)
    if norm:
        # the residual stream (updated in place by every call) and each
        # layer's norm weights
        _, r0, _ = synth.norm_inputs(1, cfg.T, cfg.H, seed=900)
        r0 = r0.to(dev)
        resid = r0.clone()
        gammas = [synth.norm_inputs(1, 1, cfg.H, seed=901 + l)[2].to(dev) for l in range(L)]
        call = lambda: ops.mxfp4_forward_layers_norm(x, layers, gammas, NORM_EPS, resid, cfg.I,
                                                     cfg.E, cfg.K, cfg.shared, cfg.act_fmt,
                                                     prefetch=pf, out=out, workspace=ws)
    else:
        call = lambda: ops.mxfp4_forward_layers(x, layers, cfg.I, cfg.E, cfg.K, cfg.shared,
                                                cfg.act_fmt, prefetch=pf, out=out, workspace=ws)
    with torch.cuda.stream(s):
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        if norm:
            resid.copy_(r0)
            call()
            torch.cuda.synchronize()
        eager_out = out.clone()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            call()
        torch.cuda.synchronize()
        eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    if norm:                              # the same residual stream as the eager call
        resid.copy_(r0)
        g.replay()
        torch.cuda.synchronize()
    if not torch.equal(out, eager_out):
        raise RuntimeError("graph replay and eager call disagree")
    log(f"{L} layers: eager {eager_ms:.4f} ms, graph {graph_ms:.4f} ms")
    res = {"metric": METRIC, "value": round(cfg.T / (graph_ms / L / 1e3), 1), "unit": "tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(graph_ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16" if cfg.act_fmt == 0 else "mxfp4",
           "data": "synthetic",
           "config": {"workload": f"{cfg.name}: {L} MoE layers in one call (T={cfg.T} H={cfg.H} "
                                  f"I={cfg.I} E={cfg.E} K={cfg.K}+{cfg.shared} shared, each routed "
                                  "from its input by its router GEMM"
                                  + (", residual add + RMSNorm after each" if norm else "")
                                  + "), one HIP graph",
                      "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "K": cfg.K,
                      "shared": cfg.shared, "layers": L, "prefetch": bool(pf), "norm": norm,
                      "parallelism": "none (1 GPU)"},
           "layers": {"L": L, "prefetch": bool(pf), "norm": norm, "eager_ms": round(eager_ms, 4),
                      "graph_ms": round(graph_ms, 4),
                      "eager_ms_per_layer": round(eager_ms / L, 4),
                      "graph_ms_per_layer": round(graph_ms / L, 4)},
           "roofline": None, "cpu_baseline": None}
    print(json.dumps(res), flush=True)


EXTRAS = ["prefill", "prefill_skewed", "w4a4"]      # timed beside the decode headline


NORM_G, NORM_H, NORM_EPS = 8, 4096, 1e-6
NORM_T = (64, 1536, 8192)          # the decode batch and the two prefill chunks


def bench_residual_norm(args, sizes=NORM_T):
    """The step after the layer at tensor-parallel degree 8, one GPU's share
    of the pages' one-shot all-reduce with the residual add and RMSNorm fused
    (VibeSys post, section "Communication and concurrency"): eight partial
    outputs [T, H] summed, the residual added, RMSNorm, per batch size T.
    args.steps back-to-back calls are captured in one HIP graph (the entry
    point allocates and synchronises nothing, so it can be captured) and the
    replay is timed with HIP events on its stream: the per-call time without
    host launch overhead.  Algorithmic bytes: the G + 1 inputs read, h and y
    written, gamma read once."""
    from mxfp4_routed_expert_top_amd import ops
    res = {}
    for T in sizes:
        p, r, g = synth.norm_inputs(NORM_G, T, NORM_H, seed=T)
        parts = [p[i].to("cuda") for i in range(NORM_G)]
        resid, gam = r.to("cuda"), g.to("cuda")
        hout, y = torch.empty_like(resid), torch.empty_like(resid)

        def call():
            ops.residual_rmsnorm(parts, gam, NORM_EPS, residual=resid, residual_out=hout, out=y)

        for _ in range(max(1, args.warmup)):
            call()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                call()
        graph.replay()                       # the first replay uploads the graph
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s = torch.cuda.current_stream()
        e0.record(s)
        graph.replay()
        e1.record(s)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        nbytes = (NORM_G + 1) * T * NORM_H * 2 + 2 * T * NORM_H * 2 + NORM_H * 2
        gbs = nbytes / (us * 1e-6) / 1e9
        res[f"T{T}"] = {"G": NORM_G, "T": T, "H": NORM_H, "us_per_call": round(us, 2),
                        "algorithmic_bytes": nbytes, "gbs": round(gbs, 1),
                        "hbm_frac": round(gbs / (HBM_PEAK_GBS), 4)}
        log(f"residual_rmsnorm T={T}: {us:.2f} us per call, {gbs:.0f} GB/s")
        del graph
    return res


def pct(a, q):
    return float(np.percentile(np.asarray(a), q))


def measure(cfg, args, weights=None, router=False):
    """One workload: whole-layer throughput over args.steps calls (wall
    clock, synchronised on both sides), the per-call HIP-event distribution,
    the GEMM kernels' durations from HIP events on their launch stream, and
    the rooflines.  Returns (result dict, weights) so a later workload with
    the same weight draw can reuse them."""
    from mxfp4_routed_expert_top_amd import ops, profiling
    w8 = cfg.wfmt == synth.W_MXFP8
    log(f"workload {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} K={cfg.K} "
        f"shared={cfg.shared} act={'mxfp4' if cfg.act_fmt else 'bf16'} "
        f"weights={'mxfp8' if w8 else 'mxfp4'}")
    x, logits, gate, *wts = make_inputs(cfg, weights)
    w13, w13s, w2, w2s = wts
    wr = synth.router_weight(cfg).to("cuda") if router else None
    if router:
        # the stage-by-stage pass routes on the logits the router GEMM gives
        lg = torch.empty(cfg.T, cfg.Ep, dtype=torch.float32, device="cuda")
        ops.route_topk_gemm(x, wr, cfg.K, cfg.shared, logits_out=lg)
        logits = lg[:, :cfg.E].contiguous()
        gate = lg[:, cfg.E].contiguous() if cfg.shared else None
    bufs = ops.alloc_stages(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, cfg.shared, cfg.act_fmt, "cuda")
    ws = torch.empty(ops.workspace_size(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K, cfg.shared, cfg.act_fmt),
                     dtype=torch.uint8, device="cuda")
    assert not w8 or ws.numel() >= ops.mxfp8_workspace_size(cfg.T, cfg.H, cfg.I, cfg.E, cfg.K,
                                                             cfg.shared)
    out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device="cuda")

    def step():
        # the whole layer, one C call: [router GEMM,] route, align, [quant x], gate/up+SwiGLU,
        # [quant h], down, combine
        if router:
            ops.mxfp4_forward_router(x, wr, w13, w13s, w2, w2s, cfg.I, cfg.E, cfg.K, cfg.shared,
                                     cfg.act_fmt, out=out, workspace=ws)
        elif w8:
            ops.mxfp8_forward(x, logits, gate, w13, w13s, w2, w2s, cfg.I, cfg.E, cfg.K,
                              cfg.shared, out=out, workspace=ws)
        else:
            ops.mxfp4_forward(x, logits, gate, w13, w13s, w2, w2s, cfg.I, cfg.E, cfg.K, cfg.shared,
                              cfg.act_fmt, out=out, workspace=ws)

    def step_stages(events):
        ops.forward_stages(x, logits, gate, w13, w13s, w2, w2s, cfg.I, cfg.E, cfg.K, cfg.shared,
                           cfg.act_fmt, bufs=bufs, events=events, wfmt=cfg.wfmt,
                           fuse_h_quant=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region 1: whole-layer throughput (no events inside the steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # two more back-to-back repeats of region 1 in the same run (paired
    # repeats show the run-to-run spread); ms_per_step stays the first
    repeats = [ms]
    for _ in range(2):
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        repeats.append((time.perf_counter() - t1) * 1e3 / args.steps)

    # timed region 2: each call between its own pair of HIP events on the
    # launch stream, for the distribution (median, p10, p90)
    stream = torch.cuda.current_stream()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    for a, b in pairs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in pairs]

    # timed region 3: the same pass stage by stage, HIP events on the launch
    # stream around the GEMM kernels (the dominant ones) for their durations
    names = ["gate_up", "down", "combine"]
    ev = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for n in names} for _ in range(args.steps)]
    for _ in range(2):
        step_stages(None)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step_stages(ev[i])
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in ev])) for n in names}
    log(f"  step {ms:.4f} ms (events: median {pct(call_ms, 50):.4f}); kernel ms:",
        json.dumps({k: round(v, 4) for k, v in stage_ms.items()}))
    if not torch.equal(out, bufs["out"]):
        raise RuntimeError("one-call forward and per-stage pass disagree")

    router_res = None
    if router:
        # timed region 4: the router call alone (router GEMM + routing), HIP events
        rws = torch.empty(ops.route_gemm_workspace_size(cfg.T, cfg.H, cfg.E, cfg.shared),
                          dtype=torch.uint8, device="cuda")
        rids = torch.empty(cfg.T, cfg.Kp, dtype=torch.int32, device="cuda")
        rw_ = torch.empty(cfg.T, cfg.Kp, dtype=torch.float32, device="cuda")
        rcall = lambda: ops.route_topk_gemm(x, wr, cfg.K, cfg.shared, topk_ids=rids,
                                            topk_weights=rw_, workspace=rws)
        for _ in range(3):
            rcall()
        # one event pair around the back-to-back calls: per-call pairs would time
        # the host whenever enqueueing a call takes longer than running it
        ra, rb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ra.record()
        for _ in range(args.steps):
            rcall()
        rb.record()
        torch.cuda.synchronize()
        rms = ra.elapsed_time(rb) / args.steps
        rbytes = cfg.Ep * cfg.H * 2 + cfg.T * cfg.H * 2
        router_res = {"call_ms": round(rms, 4), "algorithmic_bytes": rbytes,
                      "flops": 2 * cfg.T * cfg.Ep * cfg.H,
                      "gbs": round(rbytes / (rms / 1e3) / 1e9, 1)}
        log("  router call ms:", round(rms, 4))

    counts = bufs["align"]["counts"].cpu().numpy()
    alg = algorithmic(cfg, counts)
    if router:          # the router rows join the layer's bytes and FLOPs
        alg["layer_bytes"] += cfg.Ep * cfg.H * 2 - cfg.T * cfg.E * 4 - cfg.T * 4 * cfg.shared
        alg["flops"] += 2 * cfg.T * cfg.Ep * cfg.H
    tile_m = (ops.mxfp8_gemm_tile_m(cfg.T, cfg.Kp, cfg.Ep, cfg.H, cfg.I) if w8 else
              ops.gemm_tile_m(cfg.T, cfg.Kp, cfg.Ep, cfg.H, cfg.I, cfg.act_fmt))
    kname = gate_up_kernel_name(cfg, tile_m)
    gu_s = stage_ms["gate_up"] / 1e3
    mfma_peak = BF16_PEAK_TFLOPS if cfg.act_fmt == 0 else MXFP4_PEAK_TFLOPS
    t_hbm = alg["gate_up_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = alg["gate_up_flops"] / (mfma_peak * 1e12)
    traffic = profiling.load_traffic(traffic_path(cfg), kname)
    if t_hbm >= t_mfma:
        achieved = alg["gate_up_bytes"] / gu_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = alg["gate_up_flops"] / gu_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": mfma_peak,
                    "unit": "TFLOP/s", "frac": round(achieved / mfma_peak, 4)}
    roofline.update({"traffic": traffic, "kernel": kname,
                     "algorithmic_bytes": alg["gate_up_bytes"],
                     "algorithmic_flops": alg["gate_up_flops"],
                     "kernel_ms": round(stage_ms["gate_up"], 4)})
    layer_s = ms / 1e3
    t_l_hbm = alg["layer_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_l_mfma = alg["flops"] / (mfma_peak * 1e12)
    t_bind = max(t_l_hbm, t_l_mfma)
    t_mxfp4 = alg["flops"] / (MXFP4_PEAK_TFLOPS * 1e12)
    routed = counts[:cfg.E]
    res = {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "K": cfg.K,
           "shared": cfg.shared,
           "format": ("W8A16 MXFP8" if w8 else ("W4A16" if cfg.act_fmt == 0 else "W4A4") + " MXFP4"),
           "ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.T / layer_s, 1),
           "repeats_ms": [round(r, 4) for r in repeats],
           "repeat_spread": round(max(repeats) / min(repeats) - 1, 4),
           "call_ms": {"median": round(pct(call_ms, 50), 4), "p10": round(pct(call_ms, 10), 4),
                       "p90": round(pct(call_ms, 90), 4), "calls": len(call_ms)},
           "kernel_ms": {k: round(v, 4) for k, v in stage_ms.items()},
           "bytes": alg["layer_bytes"], "flops": alg["flops"],
           "hbm_gbs": round(alg["layer_bytes"] / layer_s / 1e9, 1),
           "hbm_frac": round(alg["layer_bytes"] / layer_s / 1e9 / HBM_PEAK_GBS, 4),
           "bf16_mfma_frac": round(alg["flops"] / layer_s / 1e12 / BF16_PEAK_TFLOPS, 5),
           "mxfp4_mfma_frac": round(alg["flops"] / layer_s / 1e12 / MXFP4_PEAK_TFLOPS, 5),
           "mxfp4_mfma_frac_ceiling": round(t_mxfp4 / t_bind, 4),
           "binding_roofline": "hbm" if t_l_hbm >= t_l_mfma else
                               ("bf16_mfma" if cfg.act_fmt == 0 else "mxfp4_mfma"),
           "binding_roofline_frac": round(t_bind / layer_s, 4),
           "down_gbs": round(alg["w2_bytes"] / (stage_ms["down"] / 1e3) / 1e9, 1),
           "experts": {"touched": alg["touched"], "routed_zero": int((routed == 0).sum()),
                       "routed_rows_min": int(routed.min()), "routed_rows_max": int(routed.max()),
                       "routed_rows_mean": round(float(routed.mean()), 2),
                       "shared_rows": int(counts[cfg.E]) if cfg.shared else 0},
           "roofline": roofline}
    if router_res is not None:
        res["router"] = router_res
    if args.sha:
        res["sha256"] = {"x": sha256_of(x), "logits": sha256_of(logits),
                         "gate": None if gate is None else sha256_of(gate)}
        if weights is None:         # the weight set is hashed once, where it is made
            res["sha256"]["weights"] = sha256_of(*wts)
    return res, wts


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(this layer is measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    cfg = synth.CONFIGS[args.workload]
    if args.layers:
        if cfg.wfmt == synth.W_MXFP8:
            print("--layers is for MXFP4 weights", file=sys.stderr)
            sys.exit(2)
        return bench_layers(cfg, args)
    w8 = cfg.wfmt == synth.W_MXFP8
    if args.router and w8:
        print("--router is for MXFP4 weights", file=sys.stderr)
        sys.exit(2)
    if args.pmc_calibrate:
        a = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")      # 1 GiB
        torch.bitwise_not(a, out=torch.empty_like(a))
        torch.cuda.synchronize()
        del a
        torch.cuda.empty_cache()
    if args.epilogue is not None:
        sizes = tuple(args.epilogue) or NORM_T
        print(json.dumps({"epilogue_residual_rmsnorm": bench_residual_norm(args, sizes)}),
              flush=True)
        return
    head, head_w = measure(cfg, args, router=args.router)
    extras = {}
    want_extras = (not args.no_extras and args.workload == "decode" and not args.router)
    if want_extras:
        kept = {(cfg.seed_w, cfg.H, cfg.I, cfg.E, cfg.shared, cfg.wfmt): head_w}
        for name in EXTRAS:
            c = synth.CONFIGS[name]
            key = (c.seed_w, c.H, c.I, c.E, c.shared, c.wfmt)
            r, w = measure(c, args, weights=kept.get(key))
            kept.setdefault(key, w)
            extras[name] = r
    epilogue = bench_residual_norm(args) if want_extras else None
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, router=args.router)
        log("cpu_baseline:", json.dumps(cpu))
    roofline = head.pop("roofline")
    res = {"metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": head["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if cfg.act_fmt == 0 else "mxfp4",
           "data": "synthetic",
           "config": {"workload": f"{cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} "
                                  f"K={cfg.K}+{cfg.shared} shared, {head['format']} weights"
                                  + (", routed from x by the router GEMM" if args.router else ""),
                      "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "K": cfg.K,
                      "shared": cfg.shared, "parallelism": "none (1 GPU)"},
           "roofline": roofline, "layer": head, "cpu_baseline": cpu}
    if extras:
        res["workloads"] = extras
    if epilogue:
        res["epilogue_residual_rmsnorm"] = epilogue
    if "router" in head:
        res["router"] = head.pop("router")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
