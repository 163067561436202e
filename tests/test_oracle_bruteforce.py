"""Pin the fp64 oracle against a brute force in 50-digit arithmetic.

The brute force (oracle/bruteforce.py) is a separate implementation of the
plain definitions with no max-subtraction; agreement to 1e-12 on tiny inputs
pins every step of the oracle's attention, LSE, lazy-ratio, streaming and
decode arithmetic (press-release page, "LightTransfer method": the ratio is
the attention mass on the initial and recent keys; Chinese write-up,
"solution 1": the LSE is its denominator).
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle import bruteforce as bf

TOL = 1e-12


def _mp2np(x):
    return np.array(x, dtype=np.float64)


CASES = [
    # B, N, Hq, Hkv, D, S, R, W, seed
    (1, 6, 2, 1, 3, 1, 2, 3, 0),
    (1, 9, 4, 2, 4, 2, 3, 9, 1),
    (2, 7, 2, 2, 2, 0, 1, 4, 2),
    (1, 10, 4, 1, 3, 3, 4, 5, 3),
    (1, 8, 1, 1, 4, 10, 10, 8, 4),   # S + R >= N
    (1, 12, 2, 1, 2, 1, 1, 1, 5),    # R = 1: sink + diagonal only
]


@pytest.mark.parametrize("B,N,Hq,Hkv,D,S,R,W,seed", CASES)
def test_prefill_matches_bruteforce(B, N, Hq, Hkv, D, S, R, W, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, D)) * 1.5
    k = rng.standard_normal((B, Hkv, N, D)) * 1.5
    v = rng.standard_normal((B, Hkv, N, D))
    got = oracle.prefill(q, k, v, S=S, R=R, W=W, streaming=True)
    want = bf.attention(q.tolist(), k.tolist(), v.tolist(), S=S, R=R, W=W)
    for key in ("out", "lse", "sout", "slse", "lazy_rows", "lazy_ratio"):
        np.testing.assert_allclose(got[key], _mp2np(want[key]), rtol=0, atol=TOL, err_msg=key)


def test_custom_scale_matches_bruteforce():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 2, 5, 3))
    k = rng.standard_normal((1, 1, 5, 3))
    v = rng.standard_normal((1, 1, 5, 3))
    got = oracle.prefill(q, k, v, S=1, R=2, W=2, scale=0.7)
    want = bf.attention(q.tolist(), k.tolist(), v.tolist(), S=1, R=2, W=2, scale=0.7)
    np.testing.assert_allclose(got["lse"], _mp2np(want["lse"]), atol=TOL)
    np.testing.assert_allclose(got["lazy_ratio"], _mp2np(want["lazy_ratio"]), atol=TOL)


@pytest.mark.parametrize("B,Hq,Hkv,L,D,seed", [(1, 2, 1, 1, 3, 0), (2, 4, 2, 7, 4, 1), (1, 3, 3, 11, 2, 2)])
def test_decode_matches_bruteforce(B, Hq, Hkv, L, D, seed):
    rng = np.random.default_rng(100 + seed)
    q = rng.standard_normal((B, Hq, D)) * 2
    k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, D))
    got = oracle.decode(q, k, v)
    want = bf.decode(q.tolist(), k.tolist(), v.tolist())
    np.testing.assert_allclose(got["out"], _mp2np(want["out"]), atol=TOL)
    np.testing.assert_allclose(got["lse"], _mp2np(want["lse"]), atol=TOL)


def test_rows_matches_full_prefill():
    rng = np.random.default_rng(7)
    N, D = 40, 5
    q = rng.standard_normal((1, 1, N, D))
    k = rng.standard_normal((1, 1, N, D))
    v = rng.standard_normal((1, 1, N, D))
    full = oracle.prefill(q, k, v, S=2, R=5, W=N, streaming=True)
    pos = [0, 3, 17, 39]
    r = oracle.rows(k[0, 0], v[0, 0], pos, q[0, 0, pos], S=2, R=5)
    np.testing.assert_array_equal(r["out"], full["out"][0, 0, pos])
    np.testing.assert_array_equal(r["lse"], full["lse"][0, 0, pos])
    np.testing.assert_array_equal(r["lazy"], full["lazy_rows"][0, 0, pos])
    np.testing.assert_array_equal(r["sout"], full["sout"][0, 0, pos])
