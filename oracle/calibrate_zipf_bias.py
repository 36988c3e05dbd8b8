#!/usr/bin/env python3
"""Writes gen/zipf_bias.json: the router bias of the Zipf-skewed prefill
workload (2048 bf16 tokens of the GLM-scale layer), by popularity rank.

Recipe.  "Zipf(s = 1.1) popularity" cannot hold for assignments (rank 1 would
need more slots than there are tokens), so the target is a per-token selection
probability P_r = min(1, c r^-s) with sum_r P_r = top_k (gen.zipf_targets);
ranks go to experts through the layer's seeded permutation (gen.zipf_ranks).
The bias is fitted on the workload's own tokens with the sign-update rule of
auxiliary-loss-free load balancing (DeepSeek-V3 technical report, section
2.1.2: after each step b_e moves by a fixed gamma towards balance), pointed at
the Zipf loads 2048 * P_r instead of uniform ones: b_e += gamma * sign(target_e
- load_e), gamma = 1e-3, 2000 iterations, logits computed once in fp64 by the
oracle and the selection rerun by the oracle each iteration.  The bias is
stored as float32, together with the realised loads by rank.

Run from the repository root after building the oracle:
    python oracle/calibrate_zipf_bias.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import gen  # noqa: E402
import oracle  # noqa: E402

GAMMA, ITERS = 1e-3, 2000


def main():
    cfg = gen.get_config("c3", bias=None)
    T, E, K = cfg.batches[0], cfg.n_experts, cfg.top_k
    w, _ = gen.router(cfg, 0)
    x = gen.x_tokens(cfg, T)
    d = oracle.Desc.from_config(cfg)
    z = oracle.logits(d, w, x, T)
    rank = gen.zipf_ranks(cfg, 0)
    target = T * gen.zipf_targets(E, K, cfg.zipf_s)[rank - 1]
    b = np.zeros(E, dtype=np.float64)
    for it in range(ITERS):
        idx, _, _ = oracle.select(d, z, b.astype(np.float32), T)
        load = np.bincount(idx.ravel(), minlength=E)
        b += GAMMA * np.sign(target - load)
    b32 = b.astype(np.float32)
    idx, _, _ = oracle.select(d, z, b32, T)
    load = np.bincount(idx.ravel(), minlength=E)
    by_rank = np.empty(E, dtype=np.float32)
    by_rank[rank - 1] = b32
    load_by_rank = np.empty(E, dtype=np.int64)
    load_by_rank[rank - 1] = load
    doc = {
        "n_experts": E, "top_k": K, "s": cfg.zipf_s, "tokens": T, "seed": cfg.seed,
        "gamma": GAMMA, "iterations": ITERS,
        "bias_by_rank": [float(v) for v in by_rank],
        "realized_load_by_rank": [int(v) for v in load_by_rank],
        "target_load_by_rank": [float(v) for v in T * gen.zipf_targets(E, K, cfg.zipf_s)],
        "n_active": int((load > 0).sum()),
    }
    path = os.path.join(ROOT, "gen", "zipf_bias.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
    print(f"wrote {path}: n_active {doc['n_active']}, loads by rank 1..8 "
          f"{load_by_rank[:8].tolist()} (targets {np.round(doc['target_load_by_rank'][:8], 1)})")


if __name__ == "__main__":
    main()
