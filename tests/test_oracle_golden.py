"""The oracle against stored brute-force values (tests/golden/, written by
tests/golden/make_golden.py from oracle/bruteforce.py only)."""
import json
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_golden():
    with open(os.path.join(HERE, "golden", "tiny_bruteforce.json")) as f:
        g = json.load(f)
    r = oracle.prefill(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), S=g["S"], R=g["R"],
                       W=g["W"], streaming=True)
    for key, want in g["expected"].items():
        want = np.array(want, dtype=np.float64)
        np.testing.assert_allclose(r[key], want, rtol=0, atol=1e-13, err_msg=key)
