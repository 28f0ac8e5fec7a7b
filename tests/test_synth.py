"""The seeded input generators: determinism, shapes and the skewed load."""
import math

import numpy as np
import torch

import synth
from oracle import moe


def test_deterministic_and_shaped():
    cfg = synth.CONFIGS["tiny"]
    a, b = synth.activations(cfg), synth.activations(cfg)
    assert a.dtype == torch.bfloat16 and a.shape == (cfg.T, cfg.H) and torch.equal(a, b)
    assert torch.equal(synth.router_logits(cfg), synth.router_logits(cfg))
    assert synth.gate_logits(cfg) is None
    w = synth.expert_w13(cfg, 3)
    assert w.shape == (2 * cfg.I, cfg.H) and torch.equal(w, synth.expert_w13(cfg, 3))
    assert not torch.equal(w, synth.expert_w13(cfg, 4))
    assert abs(float(w.std()) - 0.02) < 0.002


def test_outliers_present_in_w4a4_activations():
    cfg = synth.custom_config(T=512, H=1024, outlier_p=0.001)
    x = synth.activations(cfg).float()
    frac = float((x.abs() > 8).float().mean())
    assert 0.0005 < frac < 0.0015


def test_skewed_load_share_and_dead_experts():
    cfg = synth.CONFIGS["prefill_skewed"]
    ids, _ = moe.route(synth.router_logits(cfg).numpy(), None, cfg.K, 0)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    share = np.sort(counts)[::-1][: math.ceil(0.05 * cfg.E)].sum() / ids.size
    assert abs(share - 0.40) <= 0.01
    _, dead = synth.skew_bias(cfg)
    assert dead.numel() == 3 and np.all(counts[dead.numpy()] == 0)
    assert (counts == 0).sum() == 3
