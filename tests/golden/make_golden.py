"""Writes tests/golden/oracle_tiny.json: oracle outputs on tiny fixed inputs.

Calls only the oracle (oracle/). The pages print no worked numeric example, so
this fixture is a regression snapshot of the pinned oracle, not an independent
pin: a change to the oracle's arithmetic must regenerate it, and the commit that
does so names the passage (or the reading of it) that justifies the change.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def inputs():
    # small integers / 8: exact in bf16 and fp32, readable in the fixture
    rng = np.random.default_rng(2024)
    shape = (1, 2, 6, 4)
    return {n: (rng.integers(-16, 17, size=shape) / 8.0) for n in ("q", "k", "v", "do")}


CASES = {
    "dense": dict(causal=False, kv_len=None, block_mask=None, mask_block=1),
    "causal": dict(causal=True, kv_len=None, block_mask=None, mask_block=1),
    "padding": dict(causal=False, kv_len=[4], block_mask=None, mask_block=1),
    "block": dict(causal=False, kv_len=None, block_mask=[[1, 0, 1], [0, 1, 1], [1, 0, 0]], mask_block=2),
}


def main():
    x = inputs()
    out = {"inputs": {k: v.tolist() for k, v in x.items()}, "scale": 0.5, "cases": {}}
    for name, c in CASES.items():
        bm = None if c["block_mask"] is None else np.array(c["block_mask"])
        o, lse = oracle.attention_forward(x["q"], x["k"], x["v"], 0.5, causal=c["causal"], kv_len=c["kv_len"],
                                          block_mask=bm, mask_block=c["mask_block"])
        dq, dk, dv = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], 0.5, causal=c["causal"],
                                               kv_len=c["kv_len"], block_mask=bm, mask_block=c["mask_block"])
        out["cases"][name] = {"params": c, "o": o.tolist(), "lse": lse.tolist(),
                              "dq": dq.tolist(), "dk": dk.tolist(), "dv": dv.tolist()}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
