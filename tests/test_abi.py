"""C-ABI contract, on the CPU (no GPU needed, no kernel launched).

* liblt.so loads and exports every function include/lt.h declares;
* every validation error returns its status before anything is launched;
* the host-side lazy-layer queue and KV accounting agree bit for bit with
  the oracle on the same fp32 inputs.
"""
import ctypes
import math
import os
import random
import re

import numpy as np
import torch
import pytest

import oracle
from kv_cache_compression_causal_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from kv_cache_compression_causal_amd import build
        build.build()
    return _lib.lib()


def header_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(lt_[a-z0-9_]+)\s*\(", text))
    return names


def test_exports_every_declared_function(L):
    names = header_functions()
    assert names == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


V = _lib.LtView
GOOD = 0x100000  # aligned stand-in pointer; never dereferenced (validation fails first)


def view(ptr=GOOD, sb=1 << 20, sh=1 << 16, sn=128):
    return V(ptr, sb, sh, sn)


def shape(**kw):
    d = dict(B=1, N=64, Hq=4, Hkv=2, D=128, dtype=_lib.LT_BF16, scale=0.0)
    d.update(kw)
    return _lib.LtShape(**d)


def prefill(L, shp, q=None, k=None, v=None, o=None, lse=GOOD, S=4, R=8, W=4, rows=GOOD, ratio=GOOD):
    return L.lt_prefill_attn_lse_lazy(ctypes.byref(shp) if shp is not None else None,
                                      q or view(), k or view(), v or view(), o or view(),
                                      lse, S, R, W, rows, ratio, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), _lib.LT_ERR_DTYPE),
    (dict(D=96), _lib.LT_ERR_DTYPE),
    (dict(Hq=5, Hkv=2), _lib.LT_ERR_SHAPE),
    (dict(N=0), _lib.LT_ERR_SHAPE),
    (dict(B=0), _lib.LT_ERR_SHAPE),
    (dict(scale=float("nan")), _lib.LT_ERR_VALUE),
    (dict(scale=float("inf")), _lib.LT_ERR_VALUE),
    (dict(N=1 << 24, Hq=256, Hkv=1), _lib.LT_ERR_SHAPE),    # N * group size overflows int
    (dict(B=1 << 14, N=1 << 20, Hq=32), _lib.LT_ERR_SHAPE),  # B * Hq * N > 2^38
])
def test_prefill_shape_errors(L, kw, code):
    assert prefill(L, shape(**kw)) == code
    assert L.lt_last_error().decode() != ""


def test_prefill_argument_errors(L):
    s = shape()
    assert prefill(L, None) == _lib.LT_ERR_NULL
    assert prefill(L, s, q=view(ptr=0)) == _lib.LT_ERR_NULL
    assert prefill(L, s, k=view(ptr=GOOD + 2)) == _lib.LT_ERR_LAYOUT
    assert prefill(L, s, v=view(sn=130)) == _lib.LT_ERR_LAYOUT
    assert prefill(L, s, o=view(sb=-8)) == _lib.LT_ERR_LAYOUT
    assert prefill(L, s, k=view(sn=(1 << 25) + 8)) == _lib.LT_ERR_LAYOUT  # row stride limit
    assert prefill(L, s, k=view(sn=1 << 25), R=0) == _lib.LT_ERR_SHAPE    # at the limit: accepted
    assert prefill(L, s, lse=None) == _lib.LT_ERR_NULL
    assert prefill(L, s, W=65) == _lib.LT_ERR_SHAPE
    assert prefill(L, s, W=-1) == _lib.LT_ERR_SHAPE
    assert prefill(L, s, R=0) == _lib.LT_ERR_SHAPE
    assert prefill(L, s, S=-1) == _lib.LT_ERR_SHAPE
    assert prefill(L, s, S=1 << 30, R=1) == _lib.LT_ERR_SHAPE   # S + R past 2^30
    assert prefill(L, s, S=(1 << 30) - 1, R=1, rows=None) == _lib.LT_ERR_NULL  # at the limit: accepted
    assert prefill(L, s, rows=None) == _lib.LT_ERR_NULL
    assert prefill(L, s, ratio=None) == _lib.LT_ERR_NULL
    # fp32 allows strides that are multiples of 4 elements
    assert prefill(L, shape(dtype=_lib.LT_F32), v=view(sn=132), R=0) == _lib.LT_ERR_SHAPE


def test_streaming_errors(L):
    s = shape()
    f = L.lt_streaming_attn
    assert f(None, view(), view(), view(), view(), None, 4, 8, None) == _lib.LT_ERR_NULL
    assert f(ctypes.byref(s), view(), view(), view(), view(), None, 4, 0, None) == _lib.LT_ERR_SHAPE
    assert f(ctypes.byref(s), view(ptr=GOOD + 8), view(), view(), view(), None, 4, 8, None) == _lib.LT_ERR_LAYOUT


def test_decode_errors(L):
    n = ctypes.c_size_t()
    assert L.lt_hybrid_decode_workspace_bytes(8, 40, 8, 128, 100000, ctypes.byref(n)) == 0
    need = n.value
    assert need > 0
    f = L.lt_hybrid_decode_attn
    args = lambda **kw: dict(dict(B=8, Hq=40, Hkv=8, D=128, dt=_lib.LT_BF16, sc=0.0, q=GOOD, k=view(),
                                  v=view(), L=100000, o=GOOD, lse=None, ws=GOOD, wsb=need), **kw)

    def call(**kw):
        a = args(**kw)
        return f(a["B"], a["Hq"], a["Hkv"], a["D"], a["dt"], a["sc"], a["q"], a["k"], a["v"], a["L"],
                 a["o"], a["lse"], a["ws"], a["wsb"], None)
    assert call(wsb=need - 1) == _lib.LT_ERR_WORKSPACE
    assert call(ws=None) == _lib.LT_ERR_NULL
    assert call(Hq=41) == _lib.LT_ERR_SHAPE
    assert call(L=0) == _lib.LT_ERR_SHAPE
    assert call(D=80) == _lib.LT_ERR_DTYPE
    assert call(dt=3) == _lib.LT_ERR_DTYPE
    assert call(q=GOOD + 4) == _lib.LT_ERR_LAYOUT
    assert call(k=view(sn=100)) == _lib.LT_ERR_LAYOUT
    assert call(sc=float("nan")) == _lib.LT_ERR_VALUE


def test_compact_errors(L):
    f = L.lt_compact_kv_streaming
    assert f(view(), view(), view(), view(), 1, 8, 100, 128, _lib.LT_BF16, 4, 0, None) == _lib.LT_ERR_SHAPE
    assert f(view(), view(), view(ptr=0), view(), 1, 8, 100, 128, _lib.LT_BF16, 4, 10, None) == _lib.LT_ERR_NULL
    assert f(view(), view(), view(), view(), 1, 8, 100, 48, _lib.LT_BF16, 4, 10, None) == _lib.LT_ERR_DTYPE


def test_status_strings(L):
    assert [L.lt_status_str(i).decode() for i in range(8)] == [
        "LT_OK", "LT_ERR_NULL", "LT_ERR_SHAPE", "LT_ERR_DTYPE", "LT_ERR_LAYOUT", "LT_ERR_WORKSPACE",
        "LT_ERR_HIP", "LT_ERR_VALUE"]


@pytest.mark.parametrize("policy", [_lib.LT_EVICT_AFTER_PUSH, _lib.LT_EVICT_BEFORE_PUSH])
@pytest.mark.parametrize("seed", range(50))
def test_select_matches_oracle_bit_exact(L, seed, policy):
    from kv_cache_compression_causal_amd import api
    rnd = random.Random(seed)
    Lyr = rnd.randint(1, 64)
    n = rnd.randint(1, 40)
    C = rnd.randint(0, Lyr)
    hr = np.array([[rnd.choice([rnd.random(), 0.5, 0.25]) for _ in range(n)] for _ in range(Lyr)],
                  dtype=np.float32)
    score, ev, st = api.lt_select_lazy_layers(hr, C, policy)
    want_scores = [oracle.layer_score(row.astype(np.float64)) for row in hr]
    assert list(score) == want_scores
    wev, wst = oracle.select_lazy_layers(
        want_scores, C, policy="before" if policy == _lib.LT_EVICT_BEFORE_PUSH else "after")
    assert list(ev) == wev and list(st) == wst
    q = api.LazyQueue(Lyr, C, policy)
    assert [q.push(l, s) for l, s in enumerate(want_scores)] == wev
    q.close()
    q = api.LazyQueue(Lyr, C, policy)
    pushed = [q.push_ratios(l, row) for l, row in enumerate(hr)]
    assert [e for e, _ in pushed] == wev and [s for _, s in pushed] == want_scores
    q.close()
    if policy == _lib.LT_EVICT_AFTER_PUSH:  # the policy-free entry points are the default
        n_ = ctypes.c_int()
        s2, ev2, st2 = np.empty(Lyr), np.empty(Lyr, dtype=np.int32), np.empty(Lyr, dtype=np.uint8)
        assert L.lt_select_lazy_layers(
            hr.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), Lyr, n, C,
            s2.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
            ev2.ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
            st2.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))) == 0
        assert list(ev2) == wev


def test_queue_errors(L):
    from kv_cache_compression_causal_amd import api
    with pytest.raises(_lib.LtError) as e:
        api.lt_select_lazy_layers(np.array([[0.1], [float("nan")]], dtype=np.float32), 1)
    assert e.value.status == _lib.LT_ERR_VALUE
    with pytest.raises(_lib.LtError):
        api.lt_select_lazy_layers(np.zeros((3, 2), dtype=np.float32), 4)
    q = api.LazyQueue(3, 1)
    q.push(0, 0.5)
    with pytest.raises(_lib.LtError):
        q.push(2, 0.5)       # out of order
    with pytest.raises(_lib.LtError):
        q.push(1, math.inf)  # not finite
    with pytest.raises(_lib.LtError):
        api.LazyQueue(3, 4)
    with pytest.raises(_lib.LtError) as e:
        api.LazyQueue(3, 1, 7)  # unknown policy
    assert e.value.status == _lib.LT_ERR_VALUE
    with pytest.raises(_lib.LtError):
        api.lt_select_lazy_layers(np.zeros((3, 2), dtype=np.float32), 1, 2)


def test_queue_rejects_push_past_last_layer(L):
    """A queue of L layers accepts exactly the pushes 0..L-1; one more is
    LT_ERR_VALUE and leaves the queue as it was (no entry added)."""
    from kv_cache_compression_causal_amd import api
    q = api.LazyQueue(3, 1)
    evs = [q.push(l, s) for l, s in enumerate((0.5, 0.2, 0.9))]
    assert evs == oracle.select_lazy_layers([0.5, 0.2, 0.9], 1)[0]
    ev = ctypes.c_int(-7)
    assert L.lt_lazy_queue_push(q._h, 3, 0.1, ctypes.byref(ev)) == _lib.LT_ERR_VALUE
    assert ev.value == -7
    assert b"pushed" in L.lt_last_error()
    r = (ctypes.c_float * 2)(0.1, 0.2)
    assert L.lt_lazy_queue_push_ratios(q._h, 3, r, 2, None, ctypes.byref(ev)) == _lib.LT_ERR_VALUE
    q.close()


def _random_run(rnd):
    Lyr = rnd.randint(1, 40)
    C = rnd.randint(0, Lyr)
    scores = [rnd.choice([rnd.random(), 0.5, 0.25]) for _ in range(Lyr)]
    return Lyr, C, scores


@pytest.mark.parametrize("seed", range(60))
def test_kv_accounting_matches_oracle(L, seed):
    """The library's per-step KV bytes (batch call, and the online queue's
    counters after each push) equal the oracle's accounting for the same
    decisions, under both eviction timings, with and without slices written
    by the prefill."""
    from kv_cache_compression_causal_amd import api
    rnd = random.Random(7000 + seed)
    Lyr, C, scores = _random_run(rnd)
    full, stream = rnd.choice([(134217728, 4194304), (1000, 300), (8, 8), (0, 0)])
    for policy, pname in ((_lib.LT_EVICT_AFTER_PUSH, "after"), (_lib.LT_EVICT_BEFORE_PUSH, "before")):
        ev, _ = oracle.select_lazy_layers(scores, C, policy=pname)
        for emit in (False, True):
            want = oracle.kv_accounting(ev, full, stream, policy=pname, emit=emit)
            ret, tra = api.lt_kv_accounting(ev, full, stream, policy, emit)
            assert list(ret) == want["retained"] and list(tra) == want["transient"]
            q = api.LazyQueue(Lyr, C, policy)
            q.set_kv_bytes(full, stream, emit)
            got_r, got_t = [], []
            for l, sc in enumerate(scores):
                assert q.push(l, sc) == ev[l]
                r, t = q.kv_bytes()
                got_r.append(r)
                got_t.append(t)
            q.close()
            assert got_r == want["retained"] and got_t == want["transient"]


def test_kv_accounting_driver64_closed_form(L):
    """64 layers of 128 MiB full / 4 MiB streaming KV, capacity 32, layer
    scores rising with the layer index (each push evicts the new layer once
    the queue is full): all-full 8192 MiB, final 4224 MiB, peak 4348 MiB (33
    full + 31 streaming while layer 63 is added)."""
    from kv_cache_compression_causal_amd import api
    MiB = 1 << 20
    ev, _ = oracle.select_lazy_layers([l / 64 for l in range(64)], 32)
    ret, tra = api.lt_kv_accounting(ev, 128 * MiB, 4 * MiB)
    assert ret[-1] == 4224 * MiB and max(tra) == 4348 * MiB and tra[-1] == 4348 * MiB


def test_kv_accounting_errors(L):
    from kv_cache_compression_causal_amd import api
    i64 = ctypes.POINTER(ctypes.c_int64)
    ret = np.full(3, -5, dtype=np.int64)
    tra = np.full(3, -5, dtype=np.int64)
    f = L.lt_kv_accounting

    def call(ev, policy=0, full=10, stream=2, n=None):
        e = np.asarray(ev, dtype=np.int32)
        return f(e.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), len(ev) if n is None else n, policy, full, stream,
                 0, ret.ctypes.data_as(i64), tra.ctypes.data_as(i64))

    assert call([-1, 3, -1]) == _lib.LT_ERR_VALUE     # evicts a future layer
    assert call([-1, 0, 0]) == _lib.LT_ERR_VALUE      # evicts layer 0 twice
    assert call([-2, -1, -1]) == _lib.LT_ERR_VALUE
    assert call([-1, -1, -1], policy=5) == _lib.LT_ERR_VALUE
    assert call([-1, -1, -1], full=-1) == _lib.LT_ERR_VALUE
    assert call([-1, -1, -1], n=0) == _lib.LT_ERR_SHAPE
    assert list(ret) == [-5] * 3 and list(tra) == [-5] * 3   # untouched on error
    assert f(None, 3, 0, 10, 2, 0, ret.ctypes.data_as(i64), tra.ctypes.data_as(i64)) == _lib.LT_ERR_NULL
    q = api.LazyQueue(3, 1)
    r, t = ctypes.c_int64(), ctypes.c_int64()
    assert L.lt_lazy_queue_kv_bytes(q._h, ctypes.byref(r), ctypes.byref(t)) == _lib.LT_ERR_VALUE  # not set
    q.set_kv_bytes(10, 2)
    assert L.lt_lazy_queue_kv_bytes(q._h, ctypes.byref(r), ctypes.byref(t)) == _lib.LT_ERR_VALUE  # no push
    q.push(0, 0.5)
    with pytest.raises(_lib.LtError):
        q.set_kv_bytes(10, 2)   # after the first push
    assert L.lt_lazy_queue_set_kv_bytes(None, 1, 1, 0) == _lib.LT_ERR_NULL
    q.close()


@pytest.mark.parametrize("seed", range(40))
def test_select_offline_matches_oracle_bit_exact(L, seed):
    """lt_select_offline against the oracle on the same fp32 ratios: the mean
    scores bit for bit and the same streaming set (ties included)."""
    from kv_cache_compression_causal_amd import api
    rnd = random.Random(1000 + seed)
    P, Lyr, n = rnd.randint(1, 6), rnd.randint(1, 64), rnd.randint(1, 40)
    C = rnd.randint(0, Lyr)
    hr = np.array([[[rnd.choice([rnd.random(), 0.5, 0.25]) for _ in range(n)] for _ in range(Lyr)]
                   for _ in range(P)], dtype=np.float32)
    score, st = api.lt_select_offline(hr, C)
    per_prompt = [[oracle.layer_score(row.astype(np.float64)) for row in hr[p]] for p in range(P)]
    want_score, want_st = oracle.select_offline(per_prompt, C)
    assert list(score) == want_score
    assert list(st) == want_st
    if P == 1:  # one prompt: the set the push-then-pop queue keeps
        _, _, st_q = api.lt_select_lazy_layers(hr[0], C)
        assert list(st_q) == want_st


def test_select_offline_errors(L):
    from kv_cache_compression_causal_amd import api
    ok = np.full((2, 3, 4), 0.25, dtype=np.float32)
    for bad_C in (-1, 4):
        with pytest.raises(_lib.LtError) as e:
            api.lt_select_offline(ok, bad_C)
        assert e.value.status == _lib.LT_ERR_VALUE
    nan = ok.copy()
    nan[1, 2, 3] = np.nan
    st = np.full(3, 7, dtype=np.uint8)
    with pytest.raises(_lib.LtError) as e:
        api.lt_select_offline(nan, 1)
    assert e.value.status == _lib.LT_ERR_VALUE
    fp = ctypes.POINTER(ctypes.c_float)
    u8 = ctypes.POINTER(ctypes.c_uint8)
    assert L.lt_select_offline(nan.ctypes.data_as(fp), 2, 3, 4, 1, None,
                               st.ctypes.data_as(u8)) == _lib.LT_ERR_VALUE
    assert list(st) == [7, 7, 7]  # untouched on error
    assert L.lt_select_offline(ok.ctypes.data_as(fp), 0, 3, 4, 1, None,
                               st.ctypes.data_as(u8)) == _lib.LT_ERR_SHAPE
    assert L.lt_select_offline(None, 2, 3, 4, 1, None, st.ctypes.data_as(u8)) == _lib.LT_ERR_NULL
    assert L.lt_select_offline(ok.ctypes.data_as(fp), 2, 3, 4, 1, None, None) == _lib.LT_ERR_NULL


def test_varlen_errors(L):
    """The _varlen calls reject a NULL length array, then validate exactly as
    the uniform calls do (nothing is launched: every case fails first)."""
    shp = shape()
    P = ctypes.byref
    f = L.lt_prefill_attn_lse_lazy_varlen
    assert f(P(shp), None, view(), view(), view(), view(), GOOD, 4, 8, 4, GOOD, GOOD, None) == _lib.LT_ERR_NULL
    assert f(P(shape(D=96)), GOOD, view(), view(), view(), view(), GOOD, 4, 8, 4, GOOD, GOOD,
             None) == _lib.LT_ERR_DTYPE
    assert f(P(shp), GOOD, view(), view(), view(), view(), GOOD, 4, 8, 65, GOOD, GOOD, None) == _lib.LT_ERR_SHAPE
    assert f(P(shp), GOOD, view(), view(), view(), view(), None, 4, 8, 4, GOOD, GOOD, None) == _lib.LT_ERR_NULL
    assert f(P(shp), GOOD, view(sn=100), view(), view(), view(), GOOD, 4, 8, 4, GOOD, GOOD,
             None) == _lib.LT_ERR_LAYOUT
    g = L.lt_streaming_attn_varlen
    assert g(P(shp), None, view(), view(), view(), view(), None, 4, 8, None) == _lib.LT_ERR_NULL
    assert g(P(shp), GOOD, view(), view(), view(), view(), None, 4, 0, None) == _lib.LT_ERR_SHAPE
    d = L.lt_hybrid_decode_attn_varlen
    assert d(8, 40, 8, 128, _lib.LT_BF16, 0.0, GOOD, view(), view(), None, 1000, GOOD, None, GOOD, 1 << 30,
             None) == _lib.LT_ERR_NULL
    assert d(8, 40, 8, 128, _lib.LT_BF16, 0.0, GOOD, view(), view(), GOOD, 0, GOOD, None, GOOD, 1 << 30,
             None) == _lib.LT_ERR_SHAPE
    n = ctypes.c_size_t()
    assert L.lt_hybrid_decode_workspace_bytes(8, 40, 8, 128, 1000, ctypes.byref(n)) == 0
    assert d(8, 40, 8, 128, _lib.LT_BF16, 0.0, GOOD, view(), view(), GOOD, 1000, GOOD, None, GOOD,
             n.value - 16, None) == _lib.LT_ERR_WORKSPACE
    c = L.lt_compact_kv_streaming_varlen
    assert c(view(), view(), view(), view(), 1, 8, 100, 128, _lib.LT_BF16, 4, 10, None, None) == _lib.LT_ERR_NULL
    assert c(view(), view(), view(), view(), 1, 8, 100, 128, _lib.LT_BF16, 4, 0, GOOD, None) == _lib.LT_ERR_SHAPE
    a = L.lt_stream_cache_append_varlen
    assert a(view(), view(), GOOD, GOOD, 2, 2, 128, _lib.LT_BF16, 4, 60, None, None) == _lib.LT_ERR_NULL
    assert a(view(), view(), GOOD + 8, GOOD, 2, 2, 128, _lib.LT_BF16, 4, 60, GOOD, None) == _lib.LT_ERR_LAYOUT



def test_paged_decode_errors(L):
    """lt_hybrid_decode_attn_paged validates the pools, the table, the page
    geometry and the workspace (sized for max_pages * page_size keys) before
    any launch; every case below fails first."""
    f = L.lt_hybrid_decode_attn_paged
    bf = _lib.LT_BF16
    n = ctypes.c_size_t()
    assert L.lt_hybrid_decode_workspace_bytes(4, 16, 2, 128, 64 * 256, ctypes.byref(n)) == 0
    need = n.value

    def call(B=4, Hq=16, Hkv=2, D=128, dt=bf, q=GOOD, k=None, v=None, P=256, npages=300, table=GOOD,
             maxp=64, lens=GOOD, ws=GOOD, wsb=need):
        return f(B, Hq, Hkv, D, dt, 0.0, q, k or view(), v or view(), P, npages, table, maxp, lens, GOOD, None,
                 ws, wsb, None)
    assert call(table=None) == _lib.LT_ERR_NULL
    assert call(lens=None) == _lib.LT_ERR_NULL
    assert call(table=GOOD + 2) == _lib.LT_ERR_LAYOUT
    assert call(lens=GOOD + 2) == _lib.LT_ERR_LAYOUT
    for P in (8, 48, 0, -256, 1 << 21):
        assert call(P=P) == _lib.LT_ERR_SHAPE, P
    assert call(maxp=0) == _lib.LT_ERR_SHAPE
    assert call(npages=0) == _lib.LT_ERR_SHAPE
    assert call(wsb=need - 1) == _lib.LT_ERR_WORKSPACE
    assert call(D=96) == _lib.LT_ERR_DTYPE
    assert call(Hq=17) == _lib.LT_ERR_SHAPE
    assert call(k=view(sn=100)) == _lib.LT_ERR_LAYOUT
    assert call(q=None) == _lib.LT_ERR_NULL

def test_noalloc_decode_validates_before_touching_the_gpu(L):
    """lt_hybrid_decode_attn_noalloc checks its arguments, and that the
    partial states fit the library's scratch array, before anything touches
    the GPU (no GPU here: a lookup or launch would return LT_ERR_HIP)."""
    f = L.lt_hybrid_decode_attn_noalloc
    bf = _lib.LT_BF16
    n = ctypes.c_size_t()
    assert L.lt_hybrid_decode_workspace_bytes(1024, 16, 1, 128, 64, ctypes.byref(n)) == 0
    assert n.value > _lib.LT_DECODE_NOALLOC_SCRATCH_BYTES
    assert f(1024, 16, 1, 128, bf, 0.0, GOOD, view(), view(), 64, GOOD, None, None) == _lib.LT_ERR_WORKSPACE
    assert b"scratch" in L.lt_last_error()
    assert f(8, 40, 8, 96, bf, 0.0, GOOD, view(), view(), 1000, GOOD, None, None) == _lib.LT_ERR_DTYPE
    assert f(8, 40, 8, 128, bf, 0.0, GOOD, view(), view(), 0, GOOD, None, None) == _lib.LT_ERR_SHAPE
    assert f(8, 40, 8, 128, bf, 0.0, None, view(), view(), 1000, GOOD, None, None) == _lib.LT_ERR_NULL
    assert f(8, 40, 8, 128, bf, 0.0, GOOD, view(sn=100), view(), 1000, GOOD, None, None) == _lib.LT_ERR_LAYOUT


def test_kv_bytes_matches_oracle(L):
    from kv_cache_compression_causal_amd import api
    for (B, Hkv, N, D, dt, S, R) in [(1, 8, 32768, 128, 1, 4, 1020), (8, 8, 100000, 128, 1, 4, 1020),
                                     (2, 3, 10, 64, 0, 4, 20)]:
        e = 2 if dt == 1 else 4
        assert api.lt_kv_bytes(B, Hkv, N, D, dt, S, R) == oracle.kv_bytes(B, Hkv, N, D, e, S, R)


def test_probe_errors(L):
    """The measurement probes validate before any launch (no GPU call here)."""
    assert L.lt_probe_mfma_bf16(0, 1, GOOD, None) == _lib.LT_ERR_SHAPE
    assert L.lt_probe_mfma_bf16(1, 0, GOOD, None) == _lib.LT_ERR_SHAPE
    assert L.lt_probe_mfma_bf16(1, 1, None, None) == _lib.LT_ERR_NULL
    assert L.lt_probe_read(None, 16, 1, GOOD, None) == _lib.LT_ERR_NULL
    assert L.lt_probe_read(GOOD, 16, 1, None, None) == _lib.LT_ERR_NULL
    assert L.lt_probe_read(GOOD, 15, 1, GOOD, None) == _lib.LT_ERR_SHAPE
    assert L.lt_probe_read(GOOD, 0, 1, GOOD, None) == _lib.LT_ERR_SHAPE
    assert L.lt_probe_read(GOOD, 16, 0, GOOD, None) == _lib.LT_ERR_SHAPE
    assert L.lt_probe_read(GOOD + 8, 16, 1, GOOD, None) == _lib.LT_ERR_LAYOUT


def test_stream_append_errors(L):
    f = L.lt_stream_cache_append
    bf = _lib.LT_BF16
    assert f(view(), view(), GOOD, GOOD, 2, 2, 128, 5, 4, 60, 10, None) == _lib.LT_ERR_DTYPE
    assert f(view(), view(), GOOD, GOOD, 2, 2, 96, bf, 4, 60, 10, None) == _lib.LT_ERR_DTYPE
    assert f(view(), view(), GOOD, GOOD, 0, 2, 128, bf, 4, 60, 10, None) == _lib.LT_ERR_SHAPE
    assert f(view(), view(), GOOD, GOOD, 2, 2, 128, bf, -1, 60, 10, None) == _lib.LT_ERR_SHAPE
    assert f(view(), view(), GOOD, GOOD, 2, 2, 128, bf, 4, 0, 10, None) == _lib.LT_ERR_SHAPE
    assert f(view(), view(), GOOD, GOOD, 2, 2, 128, bf, 4, 60, -1, None) == _lib.LT_ERR_SHAPE
    assert f(view(), view(), None, GOOD, 2, 2, 128, bf, 4, 60, 10, None) == _lib.LT_ERR_NULL
    assert f(view(), view(), GOOD + 8, GOOD, 2, 2, 128, bf, 4, 60, 10, None) == _lib.LT_ERR_LAYOUT
    assert f(view(ptr=GOOD + 8), view(), GOOD, GOOD, 2, 2, 128, bf, 4, 60, 10, None) == _lib.LT_ERR_LAYOUT


def test_binding_refuses_host_tensors_and_bad_lazy_buffers():
    """The Python binding checks, before any call, that tensors live on the
    GPU (a host pointer reaching a kernel would fault) and that the lazy
    outputs have the shapes the kernels write."""
    from kv_cache_compression_causal_amd import api
    B, Hq, Hkv, N, D, W = 1, 4, 2, 64, 128, 8
    q = torch.zeros(B, Hq, N, D, dtype=torch.bfloat16)
    k = torch.zeros(B, Hkv, N, D, dtype=torch.bfloat16)
    out = torch.zeros_like(q)
    lse = torch.zeros(B, Hq, N)
    rows, ratio = torch.zeros(B, Hq, W), torch.zeros(B, Hq)
    with pytest.raises(ValueError, match="on the GPU"):
        api.lt_prefill_attn_lse_lazy(q, k, k, out, lse, 4, 8, W, rows, ratio)
    with pytest.raises(ValueError, match="lazy_rows"):
        api.lt_prefill_attn_lse_lazy(q, k, k, out, lse, 4, 8, W, torch.zeros(B, Hq, W - 1), ratio)
    with pytest.raises(ValueError, match="lazy_ratio"):
        api.lt_prefill_attn_lse_lazy(q, k, k, out, lse, 4, 8, W, rows, torch.zeros(B, Hq, dtype=torch.float64))
    with pytest.raises(ValueError, match="on the GPU"):
        api.lt_streaming_attn(q, k, k, out, lse, 4, 8)
    with pytest.raises(ValueError, match="on the GPU"):
        api.lt_hybrid_decode_attn(q[:, :, 0].contiguous(), k, k, N, out[:, :, 0].contiguous(), None,
                                  torch.zeros(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError, match="on the GPU"):
        api.lt_compact_kv_streaming(k, k, torch.zeros(B, Hkv, 12, D, dtype=torch.bfloat16),
                                    torch.zeros(B, Hkv, 12, D, dtype=torch.bfloat16), 4, 8)


def test_lt_log_prints_calls_and_their_status():
    """With LT_LOG=1 every C-ABI call prints one line on stderr (call, sizes,
    status and message), queue pushes their decision and KV bytes; without
    it nothing is printed.  Host-only calls here: nothing is launched."""
    import subprocess
    import sys
    code = (
        "import ctypes\n"
        "from kv_cache_compression_causal_amd import _lib, api\n"
        "L = _lib.lib()\n"
        "shp = _lib.LtShape(1, 64, 4, 2, 96, _lib.LT_BF16, 0.0)\n"
        "v = _lib.LtView(0x100000, 1 << 20, 1 << 16, 128)\n"
        "print(L.lt_prefill_attn_lse_lazy(ctypes.byref(shp), v, v, v, v, 0x100000, 4, 8, 4, 0x100000, 0x100000, None))\n"
        "q = api.LazyQueue(3, 1)\n"
        "q.set_kv_bytes(100, 10)\n"
        "print(q.push(0, 0.5), q.push(1, 0.25))\n"
    )
    env = dict(os.environ, LT_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("[lt] ")]
    assert any("lt_prefill_attn_lse_lazy(" in ln and "LT_ERR_DTYPE" in ln and "D=96" in ln for ln in lines), lines
    assert any("lt_lazy_queue_push(layer=1" in ln and "evicted 0" in ln and "retained 110 transient 200" in ln for ln in lines), lines
    env["LT_LOG"] = "0"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "[lt] " not in r.stderr


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with status 2 and says so
    before touching any GPU (so this runs on the CPU)."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2, (r.returncode, r.stdout[-500:], r.stderr[-500:])
    assert "one GPU" in (r.stdout + r.stderr)

