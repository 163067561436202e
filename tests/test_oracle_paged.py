"""Pins of the oracle's decode over paged caches (decode_paged, gather_pages).

The pools are built by cutting each sequence's contiguous keys into chunks of
page_size rows and dropping the chunks into free pool slots chosen at random,
so the block table comes from that construction, not from the gather's
formula.  Checked against the 50-digit brute force on the contiguous keys,
against the per-sequence decode, for independence from pages nobody lists
and from where the pages sit in the pool, and for the documented clamps.
"""
import numpy as np

import oracle
from oracle import bruteforce

rng = np.random.default_rng(91)


def paged_from_contiguous(k, v, lens, P, extra_pages=3):
    """Pools [num_pages, Hkv, P, D] holding sequence b's rows [0, lens[b]) of
    k/v [B, Hkv, L, D] in chunks of P rows at random slots; unused slots and
    the unfilled tail of a last page hold NaN.  Returns (k_pool, v_pool,
    table [B, max_pages]); table entries past a context are -1."""
    B, Hkv, L, D = k.shape
    chunks = [(b, c) for b in range(B) for c in range(-(-lens[b] // P))]
    num_pages = len(chunks) + extra_pages
    slots = rng.permutation(num_pages)[:len(chunks)]
    max_pages = max(1, -(-max(lens) // P))
    kp = np.full((num_pages, Hkv, P, D), np.nan)
    vp = np.full((num_pages, Hkv, P, D), np.nan)
    table = np.full((B, max_pages), -1, dtype=np.int64)
    for (b, c), slot in zip(chunks, slots):
        rows = range(c * P, min((c + 1) * P, lens[b]))
        kp[slot, :, :len(rows)] = k[b][:, rows.start:rows.stop]
        vp[slot, :, :len(rows)] = v[b][:, rows.start:rows.stop]
        table[b, c] = slot
    return kp, vp, table


def test_paged_decode_matches_brute_force_on_the_contiguous_keys():
    B, Hq, Hkv, D, P = 3, 4, 2, 4, 2
    lens = [5, 1, 4]
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, 5, D))
    v = rng.standard_normal((B, Hkv, 5, D))
    kp, vp, table = paged_from_contiguous(k, v, lens, P)
    got = oracle.decode_paged(q, kp, vp, np.maximum(table, 0), lens)
    for b, n in enumerate(lens):
        bf = bruteforce.decode(q[b:b + 1].tolist(), k[b:b + 1, :, :n].tolist(), v[b:b + 1, :, :n].tolist())
        np.testing.assert_allclose(got["out"][b], np.array(bf["out"][0], dtype=float), atol=1e-12)
        np.testing.assert_allclose(got["lse"][b], np.array(bf["lse"][0], dtype=float), atol=1e-12)


def test_paged_decode_equals_the_per_sequence_decode_bit_for_bit():
    B, Hq, Hkv, D, P, L = 4, 6, 3, 8, 4, 23
    lens = [23, 17, 4, 9]
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, D))
    kp, vp, table = paged_from_contiguous(k, v, lens, P)
    got = oracle.decode_paged(q, kp, vp, np.maximum(table, 0), lens)
    want = oracle.decode_varlen(q, k, v, lens)
    np.testing.assert_array_equal(got["out"], want["out"])
    np.testing.assert_array_equal(got["lse"], want["lse"])


def test_pages_nobody_lists_and_page_placement_do_not_matter():
    B, Hq, Hkv, D, P, L = 2, 2, 1, 8, 8, 30
    lens = [30, 11]
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, D))
    kp, vp, table = paged_from_contiguous(k, v, lens, P, extra_pages=5)
    base = oracle.decode_paged(q, kp, vp, np.maximum(table, 0), lens)
    assert np.isfinite(base["out"]).all()  # the NaN in unused pages and tails was never read
    # Entries past a context point at a NaN page: still never read.
    nan_page = int(np.setdiff1d(np.arange(kp.shape[0]), table[table >= 0])[0])
    t2 = np.where(table >= 0, table, nan_page)
    again = oracle.decode_paged(q, kp, vp, t2, lens)
    np.testing.assert_array_equal(again["out"], base["out"])
    # Move every page to another slot and renumber the table.
    perm = rng.permutation(kp.shape[0])
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    moved = oracle.decode_paged(q, kp2, vp2, perm[np.maximum(table, 0)], lens)
    np.testing.assert_array_equal(moved["out"], base["out"])
    np.testing.assert_array_equal(moved["lse"], base["lse"])


def test_clamps_and_empty_contexts():
    B, Hq, Hkv, D, P = 3, 2, 1, 4, 2
    num_pages = 4
    q = rng.standard_normal((B, Hq, D))
    kp = rng.standard_normal((num_pages, Hkv, P, D))
    vp = rng.standard_normal((num_pages, Hkv, P, D))
    table = np.array([[-7, 9], [3, 0], [1, 2]])
    lens = [4, 0, 99]
    got = oracle.decode_paged(q, kp, vp, table, lens)
    # Entries out of [0, num_pages) read the nearest end of the pool.
    want0 = oracle.decode_paged(q[:1], kp, vp, [[0, 3]], [4])
    np.testing.assert_array_equal(got["out"][0], want0["out"][0])
    # An empty context: out 0, lse -inf.
    assert (got["out"][1] == 0).all() and np.isneginf(got["lse"][1]).all()
    # A length past max_pages * page_size is clamped to it.
    want2 = oracle.decode_paged(q[2:], kp, vp, table[2:], [4])
    np.testing.assert_array_equal(got["out"][2], want2["out"][0])
