"""Regression guard: the oracle still produces the stored outputs of the
tiny seeded problem in tests/golden (written by tests/golden/make_golden.py,
which calls only the oracle).  The pages print no worked example, so this is
not an external pin; the pins are in test_oracle_pins."""
import json
import os

import numpy as np

import oracle
from tests.golden.make_golden import problem

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_reproduces_stored_tiny_layer():
    want = json.load(open(os.path.join(HERE, "tiny_layer.json")))
    shape, w, batch, kp, vp = problem()
    res = oracle.layer_step(shape, w, batch, kp, vp)
    for key in ("out", "x1", "attn"):
        assert np.allclose(res[key], np.array(want[key]), rtol=1e-12, atol=1e-12), key
