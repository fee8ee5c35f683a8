"""The oracle still reproduces its recorded outputs on the tiny workload."""
import json
import math
import os

import numpy as np

import oracle
from workloads import get_config, make_config_batch


def test_tiny_oracle_record():
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")
    rec = json.load(open(path))
    cfg = get_config("tiny")
    b = make_config_batch(cfg)
    sm = float(np.float32(1.0 / math.sqrt(cfg.head_dim)))
    assert rec["sm_scale"] == sm
    o, lse = oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, cfg.num_qo_heads,
                                     cfg.num_kv_heads, cfg.causal, sm)
    assert math.isclose(float(o.sum()), rec["o_sum"], rel_tol=0, abs_tol=1e-9)
    assert math.isclose(float(np.abs(o).sum()), rec["o_abs_sum"], rel_tol=1e-13)
    assert math.isclose(float(lse.sum()), rec["lse_sum"], rel_tol=1e-13)
    for s in rec["samples"]:
        assert math.isclose(float(o[s["token"], s["head"], s["dim"]]), s["o"], rel_tol=0,
                            abs_tol=1e-13)
        assert math.isclose(float(lse[s["token"], s["head"]]), s["lse"], rel_tol=0, abs_tol=1e-13)
