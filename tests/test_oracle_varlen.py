"""Pins of the oracle's variable-length batches (padded layout: sequence b is
its first seq_lens[b] positions and is computed as if alone).

Checked against the 50-digit brute force run on each sequence by itself,
against the uniform-length batch, for independence from whatever the padding
holds, against the closed form of all-zero queries (which fixes how a
sequence shorter than W is observed), and decode against the last prefill
row of every sequence.
"""
import numpy as np
import pytest

import oracle
from oracle import bruteforce

rng = np.random.default_rng(77)


def rand(*shape):
    return rng.standard_normal(shape)


def mp_to_np(x):
    return np.array(x, dtype=np.float64)


def test_varlen_matches_brute_force_per_sequence():
    B, Hq, Hkv, N, D, S, R, W = 3, 4, 2, 7, 8, 1, 2, 3
    q, k, v = rand(B, Hq, N, D), rand(B, Hkv, N, D), rand(B, Hkv, N, D)
    lens = [7, 2, 5]
    got = oracle.prefill_varlen(q, k, v, lens, S=S, R=R, W=W, streaming=True)
    for b, n in enumerate(lens):
        w = min(W, n)
        bf = bruteforce.attention(q[b:b + 1, :, :n].tolist(), k[b:b + 1, :, :n].tolist(),
                                  v[b:b + 1, :, :n].tolist(), S=S, R=R, W=w)
        np.testing.assert_allclose(got["out"][b, :, :n], mp_to_np(bf["out"][0]), atol=1e-12)
        np.testing.assert_allclose(got["lse"][b, :, :n], mp_to_np(bf["lse"][0]), atol=1e-12)
        np.testing.assert_allclose(got["sout"][b, :, :n], mp_to_np(bf["sout"][0]), atol=1e-12)
        np.testing.assert_allclose(got["slse"][b, :, :n], mp_to_np(bf["slse"][0]), atol=1e-12)
        np.testing.assert_allclose(got["lazy_rows"][b, :, W - w:], mp_to_np(bf["lazy_rows"][0]), atol=1e-12)
        np.testing.assert_allclose(got["lazy_ratio"][b], mp_to_np(bf["lazy_ratio"][0]), atol=1e-12)
        assert np.isnan(got["lazy_rows"][b, :, :W - w]).all()
        assert np.isnan(got["out"][b, :, n:]).all() and np.isnan(got["lse"][b, :, n:]).all()


def test_uniform_lengths_equal_the_batched_prefill():
    B, Hq, Hkv, N, D = 2, 6, 3, 40, 16
    q, k, v = rand(B, Hq, N, D), rand(B, Hkv, N, D), rand(B, Hkv, N, D)
    a = oracle.prefill_varlen(q, k, v, [N] * B, S=2, R=5, W=9, streaming=True)
    b = oracle.prefill(q, k, v, S=2, R=5, W=9, streaming=True)
    for key in b:
        np.testing.assert_array_equal(a[key], b[key])


def test_padding_contents_do_not_matter():
    B, Hq, Hkv, N, D = 3, 4, 1, 33, 8
    q, k, v = rand(B, Hq, N, D), rand(B, Hkv, N, D), rand(B, Hkv, N, D)
    lens = [33, 20, 9]
    base = oracle.prefill_varlen(q, k, v, lens, S=3, R=4, W=12, streaming=True)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for b, n in enumerate(lens):
        q2[b, :, n:] = 1e3
        k2[b, :, n:] = -1e3
        v2[b, :, n:] = 7e5
    other = oracle.prefill_varlen(q2, k2, v2, lens, S=3, R=4, W=12, streaming=True)
    for key in base:
        np.testing.assert_array_equal(base[key], other[key])


@pytest.mark.parametrize("n", [1, 2, 5, 11, 12, 30])
def test_short_sequence_observes_all_its_rows(n):
    """Zero queries: every visible key has weight 1/(i+1), so a row's lazy
    value is min(S+R, i+1)/(i+1); a sequence of n < W rows averages its n rows."""
    S, R, W, N = 2, 3, 12, 30
    q = np.zeros((1, 2, N, 4))
    k, v = rand(1, 1, N, 4), rand(1, 1, N, 4)
    got = oracle.prefill_varlen(q, k, v, [n], S=S, R=R, W=W)
    w = min(W, n)
    rows = [min(S + R, i + 1) / (i + 1) for i in range(n - w, n)]
    np.testing.assert_allclose(got["lazy_rows"][0, :, W - w:], np.array([rows, rows]), atol=1e-14)
    np.testing.assert_allclose(got["lazy_ratio"][0], [np.mean(rows)] * 2, atol=1e-14)
    assert np.isnan(got["lazy_rows"][0, :, :W - w]).all()


def test_empty_sequence_and_bad_lengths():
    q, k, v = rand(2, 2, 6, 4), rand(2, 1, 6, 4), rand(2, 1, 6, 4)
    got = oracle.prefill_varlen(q, k, v, [0, 6], S=1, R=2, W=3)
    assert np.isnan(got["out"][0]).all() and np.isnan(got["lazy_ratio"][0]).all()
    assert not np.isnan(got["out"][1]).any()
    with pytest.raises(ValueError):
        oracle.prefill_varlen(q, k, v, [7, 6])
    with pytest.raises(ValueError):
        oracle.prefill_varlen(q, k, v, [-1, 6])


def test_decode_varlen_is_the_last_row_of_each_sequence():
    B, Hq, Hkv, N, D = 4, 6, 2, 25, 8
    q, k, v = rand(B, Hq, N, D), rand(B, Hkv, N, D), rand(B, Hkv, N, D)
    lens = [25, 1, 13, 0]
    pre = oracle.prefill_varlen(q, k, v, lens)
    qd = np.stack([q[b, :, max(n - 1, 0)] for b, n in enumerate(lens)])
    dec = oracle.decode_varlen(qd, k, v, lens)
    for b, n in enumerate(lens):
        if n == 0:
            assert (dec["out"][b] == 0).all() and (dec["lse"][b] == -np.inf).all()
            continue
        np.testing.assert_allclose(dec["out"][b], pre["out"][b, :, n - 1], atol=1e-13)
        np.testing.assert_allclose(dec["lse"][b], pre["lse"][b, :, n - 1], atol=1e-13)
    bf = bruteforce.decode(qd[2:3].tolist(), k[2:3, :, :13].tolist(), v[2:3, :, :13].tolist())
    np.testing.assert_allclose(dec["out"][2], mp_to_np(bf["out"][0]), atol=1e-12)
    with pytest.raises(ValueError):
        oracle.decode_varlen(qd, k, v, [26, 1, 1, 1])
