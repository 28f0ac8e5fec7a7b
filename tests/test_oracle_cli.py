"""The C++ oracle's command-line tool (oracle/moe_oracle_cli.cpp) reads the
layer's inputs from raw files and writes the same output, bit for bit, as
the library call oracle_forward through the Python wrapper; it reports its
wall time, throughput, thread count and CPU."""
import json
import os
import subprocess

import numpy as np
import torch

import synth
from oracle import _lib, moe, mxfp4, mxfp8


def _run(tmp_path, cfg, wfmt=moe.W_MXFP4):
    q = mxfp8.quantize if wfmt == moe.W_MXFP8 else mxfp4.quantize
    packed = [(*q(synth.expert_w13(cfg, e).numpy()), *q(synth.expert_w2(cfg, e).numpy()))
              for e in range(cfg.Ep)]
    x = synth.activations(cfg).view(torch.int16).numpy().view(np.uint16)
    logits = synth.router_logits(cfg).numpy()
    gate = synth.gate_logits(cfg)
    gate = None if gate is None else gate.numpy()
    files = {"x": x, "logits": logits, "w13": np.stack([p[0] for p in packed]),
             "w13s": np.stack([p[1] for p in packed]), "w2": np.stack([p[2] for p in packed]),
             "w2s": np.stack([p[3] for p in packed])}
    if gate is not None:
        files["gate"] = gate
    args = [_lib.CLI_PATH, "--T", cfg.T, "--H", cfg.H, "--I", cfg.I, "--E", cfg.E, "--K", cfg.K,
            "--shared", cfg.shared, "--act", "mxfp4" if cfg.act_fmt else "bf16",
            "--wfmt", "mxfp8" if wfmt == moe.W_MXFP8 else "mxfp4", "--threads", 3,
            "--out", tmp_path / "out.bin"]
    for k, v in files.items():
        path = tmp_path / f"{k}.bin"
        np.ascontiguousarray(v).tofile(path)
        args += [f"--{k}", path]
    _lib.lib()                                    # builds the tool if it is missing
    r = subprocess.run([str(a) for a in args], capture_output=True, text=True, check=True)
    info = json.loads(r.stdout)
    got = np.fromfile(tmp_path / "out.bin", dtype=np.uint16).reshape(cfg.T, cfg.H)
    want = moe.forward(x, logits, gate, lambda e: packed[e], cfg.I, cfg.E, cfg.K, cfg.shared,
                       cfg.act_fmt, wfmt=wfmt)
    return got, want, info


def test_cli_matches_library_w4a16(tmp_path):
    cfg = synth.custom_config("cli", T=9, H=128, I=64, E=6, K=2, shared=1)
    got, want, info = _run(tmp_path, cfg)
    assert np.array_equal(got, want["out"])
    assert info["threads"] == 3 and info["seconds"] > 0 and info["tokens_per_s"] > 0
    assert "cpu" in info


def test_cli_matches_library_w4a4_and_mxfp8(tmp_path):
    cfg = synth.custom_config("cli4", T=5, H=64, I=64, E=4, K=1, shared=0,
                              act_fmt=synth.ACT_MXFP4, outlier_p=0.05)
    got, want, _ = _run(tmp_path, cfg)
    assert np.array_equal(got, want["out"])
    cfg8 = synth.custom_config("cli8", T=5, H=64, I=64, E=4, K=2, shared=1)
    os.makedirs(tmp_path / "m8", exist_ok=True)
    got, want, _ = _run(tmp_path / "m8", cfg8, wfmt=moe.W_MXFP8)
    assert np.array_equal(got, want["out"])


def test_thread_count_does_not_change_results():
    cfg = synth.custom_config("thr", T=17, H=128, I=96, E=5, K=2, shared=1)
    packed = [(*mxfp4.quantize(synth.expert_w13(cfg, e).numpy()),
               *mxfp4.quantize(synth.expert_w2(cfg, e).numpy())) for e in range(cfg.Ep)]
    x = synth.activations(cfg).view(torch.int16).numpy().view(np.uint16)
    l, g = synth.router_logits(cfg).numpy(), synth.gate_logits(cfg).numpy()
    outs = [moe.forward(x, l, g, lambda e: packed[e], cfg.I, cfg.E, cfg.K, 1, threads=t,
                        return_h=True) for t in (1, 2, 5)]
    for o in outs[1:]:
        assert np.array_equal(o["out_f64"], outs[0]["out_f64"])
        assert np.array_equal(o["h"], outs[0]["h"])
