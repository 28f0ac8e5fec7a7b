"""Find the popularity exponent of the skewed router bias by bisection.

TEST INFRASTRUCTURE (calls only oracle/ and the seeded draws in synth/).
The skewed prefill workload wants its most-loaded 5% of experts to take about
40% of the routed assignments (router-load imbalance; MiniMax M3 on MI355X
post, section "Optimisation checklist": record routed-token-count histograms).
This script routes the workload's own draw with the oracle for a given
beta and bisects beta until the share is 40%.  The result is stored as
synth.SKEW_BETA; tests/test_synth.py re-checks the share.

usage: python -m oracle.calibrate_skew
"""
import math

import numpy as np

import synth
from oracle import moe


def top_share(cfg, beta) -> float:
    logits = synth.router_logits(cfg, beta).numpy()
    ids, _ = moe.route(logits, None, cfg.K, 0)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    n_top = math.ceil(0.05 * cfg.E)
    return float(np.sort(counts)[::-1][:n_top].sum() / ids.size)


def main():
    cfg = synth.CONFIGS["prefill_skewed"]
    lo, hi = 0.0, 2.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if top_share(cfg, mid) < 0.40:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi), 4)
    print(f"SKEW_BETA = {beta}  (top-5% share {top_share(cfg, beta):.4f})")


if __name__ == "__main__":
    main()
