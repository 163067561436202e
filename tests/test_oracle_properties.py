"""Property tests of the oracle's attention (hypothesis): shapes, windows,
value scales and seeds are drawn at random, and each draw must satisfy what
the mathematics fixes, whatever the inputs (causal GQA prefill with LSE,
streaming attention over the sink + recent set, the lazy ratio; the
LightTransfer pages: Chinese write-up, "solution 1"; press-release page,
"LightTransfer method"):

* max_j s_ij <= LSE_i <= max_j s_ij + ln(i+1), over the visible keys j <= i;
* each output component lies within the range of the visible V rows;
* 0 <= r_i <= 1 and r_i = exp(LSE^K_i - LSE_i); LSE^K_i <= LSE_i;
* S + R >= N: the sink + recent set is every visible key, so the ratio is 1
  and streaming attention is full attention;
* the per-head ratio grows with S and with R;
* decode of the last query over the whole cache is prefill's last row.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def problems(draw):
    B = draw(st.integers(1, 2))
    Hkv = draw(st.integers(1, 3))
    G = draw(st.integers(1, 4))
    N = draw(st.integers(1, 40))
    D = draw(st.sampled_from([1, 2, 4, 8]))
    S = draw(st.integers(0, 10))
    R = draw(st.integers(1, 50))
    W = draw(st.integers(1, N))
    scale = draw(st.sampled_from([0.3, 1.0, 3.0, 8.0]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hkv * G, N, D)) * scale
    k = rng.standard_normal((B, Hkv, N, D)) * scale
    v = rng.standard_normal((B, Hkv, N, D))
    return q, k, v, S, R, W


def _scores(q, k, b, h, G):
    D = q.shape[-1]
    s = q[b, h] @ k[b, h // G].T / np.sqrt(D)
    N = s.shape[0]
    return np.where(np.tri(N, dtype=bool), s, -np.inf)


@SETTINGS
@given(problems())
def test_lse_bounds_and_output_range(p):
    q, k, v, S, R, W = p
    B, Hq, N, D = q.shape
    G = Hq // k.shape[1]
    r = oracle.prefill(q, k, v, S=S, R=R, W=W)
    for b in range(B):
        for h in range(Hq):
            mx = _scores(q, k, b, h, G).max(axis=1)
            lse = r["lse"][b, h]
            assert np.all(mx <= lse + 1e-12)
            assert np.all(lse <= mx + np.log(np.arange(1, N + 1)) + 1e-12)
            vv = v[b, h // G]
            hi = np.maximum.accumulate(vv, axis=0)
            lo = np.minimum.accumulate(vv, axis=0)
            assert np.all(r["out"][b, h] <= hi + 1e-12) and np.all(r["out"][b, h] >= lo - 1e-12)


@SETTINGS
@given(problems())
def test_ratio_is_the_lse_gap_and_lies_in_unit_interval(p):
    q, k, v, S, R, W = p
    r = oracle.prefill(q, k, v, S=S, R=R, W=W, streaming=True)
    N = q.shape[2]
    rows = r["lazy_rows"]
    assert np.all(rows >= 0.0) and np.all(rows <= 1.0 + 1e-13)
    gap = np.exp(r["slse"][:, :, N - W:] - r["lse"][:, :, N - W:])
    np.testing.assert_allclose(rows, gap, rtol=1e-10, atol=1e-13)
    assert np.all(r["slse"] <= r["lse"] + 1e-12)
    np.testing.assert_allclose(r["lazy_ratio"], rows.mean(axis=2), rtol=1e-12, atol=1e-15)


@SETTINGS
@given(problems())
def test_window_covering_everything_is_full_attention(p):
    q, k, v, S, R, W = p
    N = q.shape[2]
    R = max(R, N - S) if S < N else R
    r = oracle.prefill(q, k, v, S=S, R=R, W=W, streaming=True)
    np.testing.assert_allclose(r["lazy_ratio"], 1.0, atol=1e-12)
    assert np.array_equal(r["sout"], r["out"]) and np.array_equal(r["slse"], r["lse"])


@SETTINGS
@given(problems())
def test_ratio_grows_with_s_and_r(p):
    q, k, v, S, R, W = p
    base = oracle.prefill(q, k, v, S=S, R=R, W=W, full=False)["lazy_ratio"]
    more_s = oracle.prefill(q, k, v, S=S + 1, R=R, W=W, full=False)["lazy_ratio"]
    more_r = oracle.prefill(q, k, v, S=S, R=R + 1, W=W, full=False)["lazy_ratio"]
    assert np.all(more_s >= base - 1e-14) and np.all(more_r >= base - 1e-14)


@SETTINGS
@given(problems())
def test_decode_is_the_last_prefill_row(p):
    q, k, v, S, R, W = p
    r = oracle.prefill(q, k, v, S=S, R=R, W=W)
    d = oracle.decode(np.ascontiguousarray(q[:, :, -1]), k, v)
    np.testing.assert_allclose(d["out"], r["out"][:, :, -1], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(d["lse"], r["lse"][:, :, -1], rtol=1e-12, atol=1e-13)


# The same properties as one check on fixed draws, so that they can be run
# against the planted mistakes of test_oracle_mutations: they catch every
# mutant except the two window off-by-ones, which keep every invariant (any
# sink + recent set does) and fall to the brute-force pins instead.
def _props_hold(lib) -> bool:
    rng = np.random.default_rng(11)
    for _ in range(6):
        B, Hkv, G, N, D, S, R, W = 1, 2, 2, 30, 4, 3, 7, 12
        q = rng.standard_normal((B, Hkv * G, N, D)) * 2
        k = rng.standard_normal((B, Hkv, N, D)) * 2
        v = rng.standard_normal((B, Hkv, N, D))
        r = oracle.prefill(q, k, v, S=S, R=R, W=W, streaming=True, lib=lib)
        for h in range(Hkv * G):
            mx = _scores(q, k, 0, h, G).max(axis=1)
            lse = r["lse"][0, h]
            if not (np.all(mx <= lse + 1e-12) and np.all(lse <= mx + np.log(np.arange(1, N + 1)) + 1e-12)):
                return False
            vv = v[0, h // G]
            if not (np.all(r["out"][0, h] <= np.maximum.accumulate(vv, 0) + 1e-12)
                    and np.all(r["out"][0, h] >= np.minimum.accumulate(vv, 0) - 1e-12)):
                return False
        rows = r["lazy_rows"]
        if not (np.all(rows >= 0) and np.all(rows <= 1 + 1e-13)):
            return False
        if not np.allclose(rows, np.exp(r["slse"][:, :, N - W:] - r["lse"][:, :, N - W:]), rtol=1e-10, atol=1e-13):
            return False
        if not np.all(r["slse"] <= r["lse"] + 1e-12):
            return False
        if not np.allclose(r["lazy_ratio"], rows.mean(axis=2), rtol=1e-12):
            return False
        full = oracle.prefill(q, k, v, S=S, R=N, W=W, streaming=True, lib=lib)
        if not (np.allclose(full["lazy_ratio"], 1.0, atol=1e-12) and np.array_equal(full["sout"], full["out"])):
            return False
    return True


def test_properties_hold_for_the_oracle():
    assert _props_hold(None)


CAUGHT_BY_PROPERTIES = ["dropped_scale", "gqa_map_modulo", "lazy_rows_shifted", "lse_drops_max",
                        "mean_over_w_plus_1", "normalised_by_max", "stream_lse_full_max", "wrong_k_index"]


def test_properties_catch_planted_mistakes():
    import tempfile
    import test_oracle_mutations as tm
    with open(tm.SRC) as f:
        text = f.read()
    for name in CAUGHT_BY_PROPERTIES:
        old, new = tm.MUTANTS[name]
        with tempfile.TemporaryDirectory() as tmp:
            assert not _props_hold(tm._build(text.replace(old, new), tmp)), f"mutant {name} keeps the properties"
