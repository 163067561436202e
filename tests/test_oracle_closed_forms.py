"""Pin the oracle against closed forms and invariants of the method.

Zero queries make every visible key equally weighted, so LSE_i = ln(i+1),
out_i is the prefix mean of V and the per-row lazy ratio is
|K_i| / (i+1) with |K_i| = min(i+1, S+R); the per-head ratio is their mean
over the last W rows, which is (S+R)/N for W = 1 (press-release page,
"LightTransfer method", for the ratio; the sink + recent set is read as
j < S or i-R < j <= i).
"""
import math

import numpy as np
import pytest

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _rho_zero_q(N, S, R, W):
    return sum(min(S + R, i + 1) / (i + 1) for i in range(N - W, N)) / W


def test_zero_queries_closed_form():
    B, N, Hq, Hkv, D, S, R, W = 1, 300, 4, 2, 8, 4, 30, 40
    q = np.zeros((B, Hq, N, D))
    k = _rand((B, Hkv, N, D), 1)
    v = _rand((B, Hkv, N, D), 2)
    r = oracle.prefill(q, k, v, S=S, R=R, W=W, streaming=True)
    i = np.arange(N)
    np.testing.assert_allclose(r["lse"], np.broadcast_to(np.log(i + 1.0), (B, Hq, N)), atol=1e-12)
    prefix_mean = np.cumsum(v, axis=2) / (i + 1.0)[None, None, :, None]
    G = Hq // Hkv
    for h in range(Hq):
        np.testing.assert_allclose(r["out"][:, h], prefix_mean[:, h // G], atol=1e-12)
    want_rows = np.array([min(S + R, x + 1) / (x + 1) for x in range(N - W, N)])
    np.testing.assert_allclose(r["lazy_rows"], np.broadcast_to(want_rows, (B, Hq, W)), atol=1e-12)
    np.testing.assert_allclose(r["lazy_ratio"], _rho_zero_q(N, S, R, W), atol=1e-12)


@pytest.mark.parametrize("N,S,R,W,expected", [
    (512, 4, 60, 32, 0.12894692),       # tiny workload shape
    (8192, 4, 1020, 64, 0.12548315),    # Mistral-7B-shaped workload
])
def test_zero_query_ratio_at_workload_shapes(N, S, R, W, expected):
    """The exact zero-query ratio at the workload shapes (the W = 1 value
    (S+R)/N is only the limit; W > 1 averages rows with fewer keys)."""
    q = np.zeros((1, 1, N, 4))
    k = _rand((1, 1, N, 4), 3)
    v = _rand((1, 1, N, 4), 4)
    r = oracle.prefill(q, k, v, S=S, R=R, W=W, full=False)
    assert abs(r["lazy_ratio"][0, 0] - expected) < 5e-9
    assert abs(_rho_zero_q(N, S, R, W) - expected) < 5e-9


@pytest.mark.parametrize("N,S,R", [(100, 4, 20), (64, 0, 64), (33, 3, 5)])
def test_zero_queries_w1_is_s_plus_r_over_n(N, S, R):
    q = np.zeros((1, 2, N, 4))
    r = oracle.prefill(q, _rand((1, 1, N, 4), 5), _rand((1, 1, N, 4), 6), S=S, R=R, W=1, full=False)
    np.testing.assert_allclose(r["lazy_ratio"], min(S + R, N) / N, atol=1e-14)


def test_row_zero():
    q = _rand((1, 3, 20, 6), 7)
    k = _rand((1, 1, 20, 6), 8)
    v = _rand((1, 1, 20, 6), 9)
    r = oracle.prefill(q, k, v)
    s00 = (q[0, :, 0] @ k[0, 0, 0]) / math.sqrt(6)
    np.testing.assert_allclose(r["lse"][0, :, 0], s00, atol=1e-13)
    np.testing.assert_allclose(r["out"][0, :, 0], np.broadcast_to(v[0, 0, 0], (3, 6)), atol=1e-14)


def test_full_window_gives_ratio_one_and_streaming_equals_full():
    N = 50
    q, k, v = _rand((2, 4, N, 8), 10, 2.0), _rand((2, 2, N, 8), 11, 2.0), _rand((2, 2, N, 8), 12)
    for S, R in [(0, N), (N, 1), (10, 40), (30, 30)]:
        r = oracle.prefill(q, k, v, S=S, R=R, W=N, streaming=True)
        np.testing.assert_allclose(r["lazy_ratio"], 1.0, atol=1e-13)
        assert np.array_equal(r["sout"], r["out"])
        assert np.array_equal(r["slse"], r["lse"])


def test_invariants_random():
    N, S, R, W = 200, 4, 25, 200
    q, k, v = _rand((1, 6, N, 16), 13, 2.0), _rand((1, 3, N, 16), 14, 2.0), _rand((1, 3, N, 16), 15)
    r = oracle.prefill(q, k, v, S=S, R=R, W=W, streaming=True)
    rows = r["lazy_rows"]
    assert np.all(rows >= 0) and np.all(rows <= 1 + 1e-15)
    # r_i = exp(LSE_stream - LSE_full)
    np.testing.assert_allclose(rows, np.exp(r["slse"] - r["lse"]), rtol=1e-12, atol=1e-14)
    assert np.all(r["slse"] <= r["lse"] + 1e-13)
    # max_j s_ij <= LSE_i <= max_j s_ij + ln(i+1)
    G = 2
    for h in range(6):
        s = q[0, h] @ k[0, h // G].T / 4.0
        s = np.where(np.tri(N, dtype=bool), s, -np.inf)
        mx = s.max(axis=1)
        assert np.all(mx <= r["lse"][0, h] + 1e-13)
        assert np.all(r["lse"][0, h] <= mx + np.log(np.arange(1, N + 1)) + 1e-13)
        # out lies within the per-component range of the visible V rows
        cmax = np.maximum.accumulate(v[0, h // G], axis=0)
        cmin = np.minimum.accumulate(v[0, h // G], axis=0)
        assert np.all(r["out"][0, h] <= cmax + 1e-12) and np.all(r["out"][0, h] >= cmin - 1e-12)


def test_ratio_monotone_in_s_and_r():
    N, W = 120, 30
    q, k, v = _rand((1, 2, N, 8), 16, 2.0), _rand((1, 1, N, 8), 17, 2.0), _rand((1, 1, N, 8), 18)
    prev = None
    for S in range(0, 12, 2):
        x = oracle.prefill(q, k, v, S=S, R=10, W=W, full=False)["lazy_ratio"]
        if prev is not None:
            assert np.all(x >= prev - 1e-15)
        prev = x
    prev = None
    for R in (1, 2, 5, 10, 40, 120):
        x = oracle.prefill(q, k, v, S=4, R=R, W=W, full=False)["lazy_ratio"]
        if prev is not None:
            assert np.all(x >= prev - 1e-15)
        prev = x


def test_dominant_sink_key_drives_ratio_to_one():
    N, D = 64, 8
    u = np.ones(D) / math.sqrt(D)
    q = np.broadcast_to(u, (1, 1, N, D)).copy()
    k = _rand((1, 1, N, D), 19) * 0.1
    k[0, 0, 0] = 200.0 * u
    r = oracle.prefill(q, k, _rand((1, 1, N, D), 20), S=1, R=1, W=16, full=False)
    assert r["lazy_ratio"][0, 0] > 1 - 1e-12
    # and with no sink kept, the same rows give almost nothing
    r0 = oracle.prefill(q, k, _rand((1, 1, N, D), 20), S=0, R=1, W=16, full=False)
    assert r0["lazy_ratio"][0, 0] < 1e-12


def test_decode_equals_last_prefill_row():
    N = 70
    q, k, v = _rand((2, 4, N, 8), 21, 2.0), _rand((2, 2, N, 8), 22), _rand((2, 2, N, 8), 23)
    full = oracle.prefill(q, k, v)
    d = oracle.decode(q[:, :, N - 1], k, v)
    assert np.array_equal(d["out"], full["out"][:, :, N - 1])
    assert np.array_equal(d["lse"], full["lse"][:, :, N - 1])


def test_streaming_decode_on_compacted_cache_equals_streaming_row():
    N, S, R = 90, 4, 20
    q, k, v = _rand((1, 4, N, 8), 24, 2.0), _rand((1, 2, N, 8), 25), _rand((1, 2, N, 8), 26)
    st = oracle.prefill(q, k, v, S=S, R=R, streaming=True, full=False)
    idx = oracle.streaming_rows(N, S, R)
    assert sorted(idx) == list(range(S)) + list(range(N - R, N))
    srt = sorted(idx)
    d = oracle.decode(q[:, :, N - 1], k[:, :, srt], v[:, :, srt])
    assert np.array_equal(d["out"], st["sout"][:, :, N - 1])
    assert np.array_equal(d["lse"], st["slse"][:, :, N - 1])
    # in the cache's own (ring) slot order: equal up to summation order
    d2 = oracle.decode(q[:, :, N - 1], k[:, :, idx], v[:, :, idx])
    np.testing.assert_allclose(d2["out"], d["out"], atol=1e-12)
    np.testing.assert_allclose(d2["lse"], d["lse"], atol=1e-12)


def test_decode_slot_order_irrelevant():
    q, k, v = _rand((1, 2, 8), 27, 2.0), _rand((1, 1, 50, 8), 28), _rand((1, 1, 50, 8), 29)
    perm = np.random.default_rng(30).permutation(50)
    a = oracle.decode(q, k, v)
    b = oracle.decode(q, k[:, :, perm], v[:, :, perm])
    np.testing.assert_allclose(a["out"], b["out"], atol=1e-14)
    np.testing.assert_allclose(a["lse"], b["lse"], atol=1e-14)


def test_streaming_rows_edge_cases():
    assert oracle.streaming_rows(10, 4, 20) == list(range(10))
    assert oracle.streaming_rows(24, 4, 20) == list(range(24))
    # position 24 wraps round the ring of 20 recent slots to slot 4
    assert oracle.streaming_rows(25, 4, 20) == [0, 1, 2, 3, 24] + list(range(5, 24))
    assert oracle.streaming_rows(25, 0, 3) == [24, 22, 23]
    assert [oracle.stream_slot(p, 4, 20) for p in (0, 3, 4, 23, 24, 43, 44)] == [0, 3, 4, 23, 4, 23, 4]


@pytest.mark.parametrize("seed", range(40))
def test_stream_append_keeps_the_window(seed):
    """Compaction of N0 tokens then appends up to position P: the cache holds
    exactly the sink + recent set of P (positions [0, S) and (P-R, P]), and
    appends from an empty cache reproduce compaction's layout slot by slot."""
    rnd = np.random.default_rng(seed)
    S, R = int(rnd.integers(0, 6)), int(rnd.integers(1, 12))
    N0, T = int(rnd.integers(1, 40)), int(rnd.integers(1, 40))
    rows = oracle.streaming_rows(N0, S, R)
    for pos in range(N0, N0 + T):
        rows = oracle.stream_append(rows, pos, S, R)
        want = set(range(min(S, pos + 1))) | set(range(max(S, pos + 1 - R), pos + 1))
        assert {p for p in rows if p >= 0} == want
    fresh = []
    for pos in range(N0 + T):
        fresh = oracle.stream_append(fresh, pos, S, R)
    n = min(N0 + T, S + R)
    assert fresh[:n] == oracle.streaming_rows(N0 + T, S, R)


def test_argument_errors():
    q = np.zeros((1, 3, 4, 2))
    with pytest.raises(ValueError):
        oracle.prefill(q, np.zeros((1, 2, 4, 2)), np.zeros((1, 2, 4, 2)))  # Hq % Hkv
    with pytest.raises(ValueError):
        oracle.prefill(q, np.zeros((1, 1, 4, 2)), np.zeros((1, 1, 4, 2)), W=5)  # W > N
