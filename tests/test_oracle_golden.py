"""Regression: the oracle still reproduces its stored tiny snapshot (tests/golden/oracle_tiny.json)."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_tiny.json")


def test_oracle_matches_golden_snapshot():
    with open(GOLDEN) as f:
        g = json.load(f)
    x = {k: np.array(v) for k, v in g["inputs"].items()}
    for name, c in g["cases"].items():
        p = c["params"]
        bm = None if p["block_mask"] is None else np.array(p["block_mask"])
        o, lse = oracle.attention_forward(x["q"], x["k"], x["v"], g["scale"], causal=p["causal"],
                                          kv_len=p["kv_len"], block_mask=bm, mask_block=p["mask_block"])
        grads = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], g["scale"], causal=p["causal"],
                                          kv_len=p["kv_len"], block_mask=bm, mask_block=p["mask_block"])
        assert np.allclose(o, c["o"], rtol=0, atol=1e-14), name
        assert np.allclose(lse, np.array(c["lse"], dtype=float), rtol=0, atol=1e-14), name
        for got, key in zip(grads, ("dq", "dk", "dv")):
            assert np.allclose(got, c[key], rtol=0, atol=1e-13), (name, key)
