"""Writes tiny_oracle.json: the oracle's outputs for the tiny ragged workload
(2 requests, qo = kv = {17, 64}, 4/2 heads, hd128, causal, seed 1).

The pages print no worked numeric example for ragged prefill attention, so
this file holds no page values: it is a regression record of the pinned
oracle (pinned in tests/pins.py), written by this script, which calls only
oracle/ and workloads/.  Run: python tests/golden/make_golden.py
"""
import json
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import get_config, make_config_batch  # noqa: E402


def main():
    cfg = get_config("tiny")
    b = make_config_batch(cfg)
    sm = float(np.float32(1.0 / math.sqrt(cfg.head_dim)))
    o, lse = oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, cfg.num_qo_heads,
                                     cfg.num_kv_heads, cfg.causal, sm)
    picks = [(0, 0, 0), (5, 1, 17), (16, 3, 127), (17, 0, 3), (40, 2, 64), (80, 3, 100)]
    out = {
        "workload": cfg.description,
        "sm_scale": sm,
        "o_sum": float(o.sum()),
        "o_abs_sum": float(np.abs(o).sum()),
        "lse_sum": float(lse.sum()),
        "samples": [{"token": t, "head": h, "dim": d, "o": float(o[t, h, d]),
                     "lse": float(lse[t, h])} for t, h, d in picks],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
