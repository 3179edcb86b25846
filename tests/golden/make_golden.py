"""Writes tiny_f32_layer.json: the oracle's output on the tiny fp32 workload
(H=256, E=32, k=4, I=Is=128, seed 0, tokens 0-3, attempt 0).

The pages print no value of any intermediate of the MoE layer, so this file
is a regression fixture of the oracle, not a pin to the pages: it freezes what
the pinned oracle computes today. Only the oracle and the input generator run
here. Usage: python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
import synth  # noqa: E402
from helpers import host_layer  # noqa: E402


def compute():
    w = synth.WORKLOADS["tiny_f32"]
    L = host_layer(w)
    x = synth.x_tokens(w, 4)
    y, idx, wts, logits = oracle.layer(oracle.desc_of(w), L, x)
    return {"workload": "tiny_f32", "tokens": 4,
            "y_hex": [[float(v).hex() for v in row] for row in y],
            "idx": idx.tolist(), "w_hex": [[float(v).hex() for v in row] for row in wts],
            "logits_hex": [[float(v).hex() for v in row] for row in logits]}


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_f32_layer.json"), "w") as f:
        json.dump(compute(), f)
        f.write("\n")
