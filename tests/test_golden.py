"""The oracle's tiny fp32 layer output must not drift from the committed
fixture (tests/golden/tiny_f32_layer.json, written by make_golden.py)."""
import json
import os

import numpy as np

from golden.make_golden import compute

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_f32_fixture():
    with open(os.path.join(HERE, "golden", "tiny_f32_layer.json")) as f:
        ref = json.load(f)
    got = compute()
    assert got["idx"] == ref["idx"]
    for key in ("y_hex", "w_hex", "logits_hex"):
        a = np.array([[float.fromhex(v) for v in r] for r in got[key]])
        b = np.array([[float.fromhex(v) for v in r] for r in ref[key]])
        assert np.array_equal(a, b), key
