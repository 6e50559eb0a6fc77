"""Calibrate the scale of the Zipf logit bias of the skewed-load workload.

The workload asks for a Zipf(s) per-expert logit bias under which the hottest
expert receives roughly 10x the mean load.  The bias is b_e = -alpha * s *
ln(e + 1); this script finds alpha by bisection so that, on the seeded batch,
max_e n_e / mean_e n_e lies in [9.5, 10.5], and writes it to zipf_alpha.json.
The routing it needs comes from the oracle (CPU, fp64) only.

    python synth/calibrate_zipf.py
"""
import json
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
import synth  # noqa: E402


def load_ratio(cfg, logits, alpha):
    bias = synth.zipf_logit_bias(cfg, alpha=alpha).numpy()
    ids, _ = oracle.route_select(logits, cfg.k, oracle.SOFTMAX, renormalize=cfg.renormalize,
                                 bias=bias)
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    return counts.max() / counts.mean(), counts


def main(name="c4_qwen3_skew_bf16", target=10.0):
    cfg = synth.config(name)
    x, w_r, _ = synth.router_inputs(cfg, with_bias=False)
    as_bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    logits = oracle.router_logits(as_bits(x), as_bits(w_r))
    lo, hi = 0.0, 8.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        r, _ = load_ratio(cfg, logits, mid)
        if r < target:
            lo = mid
        else:
            hi = mid
    alpha = 0.5 * (lo + hi)
    ratio, counts = load_ratio(cfg, logits, alpha)
    assert 9.5 <= ratio <= 10.5, ratio
    path = os.path.join(HERE, "zipf_alpha.json")
    table = json.load(open(path)) if os.path.exists(path) else {}
    table[name] = {"alpha": alpha, "hot_over_mean": float(ratio),
                   "counts_head": counts[:8].tolist(), "counts_min": int(counts.min())}
    with open(path, "w") as f:
        json.dump(table, f, indent=2)
    print(name, table[name])


if __name__ == "__main__":
    main()
