"""Plain fp64 CPU oracle for the LightTransfer-Test hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library and never imports it; the product path does not
import it either.

Pieces:
  * ``liblt_oracle.so`` (built from ``lt_oracle.c`` by :func:`build`): causal
    attention with each softmax row materialised, its LSE, the per-row and
    per-head lazy ratio, streaming attention and decode -- all in double.
  * pure-Python host logic: the layer score, the lazy-layer priority queue,
    the streaming-cache row set and the KV byte accounting.

Sources (LightTransfer web pages; cited by page title and section):
  * Chinese write-up (xzbcqc.com), "solution 2": a queue keyed by lazy ratio
    is kept during prefill; once the number of queued layers exceeds the
    threshold (e.g. 50% of layers) the highest-ratio layer is removed and its
    KV cache switched to the streaming version.
  * LightTransfer project page, Figure 2 caption: the queue stores (lazy
    ratio, layer index) after each layer; the evicted layer's KV is reduced.
  * Press-release page (wuwenjie.xyz), "LightTransfer method": the lazy ratio
    sums the attention weights from queries to the initial and recent keys;
    offline, the 50% of layers with the highest ratio are replaced.

Readings where the pages are silent:
  * the queue pushes first and pops while its size exceeds the capacity, so
    the current layer can be evicted at its own step; equal scores evict the
    lower layer index first;
  * a layer's score is the mean of its per-head ratios over (batch, head);
  * a streaming cache keeps rows [0, S) and [N-R, N), sinks in their own
    slots and the recent rows in ring order (stream_slot);
  * offline selection averages each layer's score over the prompts (fp64,
    prompt order) before taking the top half.
  * a paged cache (the pages describe none) holds key j of sequence b in
    row j % page_size of pool page block_table[b][j // page_size]; decode
    over it is decode over the keys gathered that way (gather_pages).

Parity pins: tests/test_oracle_*.py (brute force in 50-digit arithmetic,
torch fp64 library routines, closed forms, invariants, exhaustive queue
checks).
"""
from __future__ import annotations

import ctypes
import heapq
import math
import os
import subprocess
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lt_oracle.c")
_LIB = os.path.join(_HERE, "liblt_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile lt_oracle.c into liblt_oracle.so with gcc and OpenMP."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """Bind the oracle's C entry points from the shared library at ``path``."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.lto_prefill.argtypes = [ctypes.c_int] * 5 + [ctypes.c_double, dp, dp, dp] + \
        [ctypes.c_int] * 3 + [dp] * 6
    lib.lto_prefill.restype = ctypes.c_int
    lib.lto_rows.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, dp, dp,
                             ctypes.c_int, ip, dp, ctypes.c_int, ctypes.c_int] + [dp] * 5
    lib.lto_rows.restype = ctypes.c_int
    lib.lto_decode.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double, dp, dp, dp,
                                                     ctypes.c_long, dp, dp]
    lib.lto_decode.restype = ctypes.c_int
    lib.lto_threads.argtypes = []
    lib.lto_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = load_library(_LIB)
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().lto_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_scale(D: int) -> float:
    """Softmax scale 1/sqrt(D) (the pages are silent; Flash Attention's default)."""
    return 1.0 / math.sqrt(D)


def prefill(q, k, v, S: int = 0, R: int = 1, W: int = 0, scale: Optional[float] = None,
            streaming: bool = False, full: bool = True, lib=None) -> Dict[str, np.ndarray]:
    """Causal GQA prefill; q [B,Hq,N,D], k/v [B,Hkv,N,D].

    Returns out/lse (if ``full``), sout/slse (if ``streaming``) and, for W > 0,
    lazy_rows [B,Hq,W] and lazy_ratio [B,Hq]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, D) and v.shape == k.shape
    sc = default_scale(D) if scale is None else float(scale)
    res: Dict[str, np.ndarray] = {}
    out = lse = sout = slse = lrows = lratio = None
    if full:
        out = np.empty((B, Hq, N, D)); lse = np.empty((B, Hq, N))
        res["out"], res["lse"] = out, lse
    if streaming:
        sout = np.empty((B, Hq, N, D)); slse = np.empty((B, Hq, N))
        res["sout"], res["slse"] = sout, slse
    if W > 0:
        lrows = np.empty((B, Hq, W)); lratio = np.empty((B, Hq))
        res["lazy_rows"], res["lazy_ratio"] = lrows, lratio
    rc = (lib or _load()).lto_prefill(B, N, Hq, Hkv, D, sc, _ptr(q), _ptr(k), _ptr(v), S, R, W,
                             _ptr(out), _ptr(lse), _ptr(sout), _ptr(slse), _ptr(lrows),
                             _ptr(lratio))
    if rc != 0:
        raise ValueError(f"lto_prefill failed with code {rc}")
    return res


def rows(k_head, v_head, positions: Sequence[int], q_rows, S: int = 0, R: int = 1,
         scale: Optional[float] = None, lazy: bool = True,
         streaming: bool = True, lib=None) -> Dict[str, np.ndarray]:
    """Selected query rows of one head.  k_head/v_head [N,D] are the head's KV;
    q_rows [n,D] are the queries at ``positions`` (each sees keys 0..pos)."""
    k_head, v_head, q_rows = _f64(k_head), _f64(v_head), _f64(q_rows)
    nk, D = k_head.shape
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32))
    n = pos.shape[0]
    assert q_rows.shape == (n, D)
    sc = default_scale(D) if scale is None else float(scale)
    out = np.empty((n, D)); lse = np.empty(n)
    lz = np.empty(n) if lazy else None
    so = np.empty((n, D)) if streaming else None
    sl = np.empty(n) if streaming else None
    rc = (lib or _load()).lto_rows(nk, D, sc, _ptr(k_head), _ptr(v_head), n,
                          pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), _ptr(q_rows),
                          S, R, _ptr(out), _ptr(lse), _ptr(lz), _ptr(so), _ptr(sl))
    if rc != 0:
        raise ValueError(f"lto_rows failed with code {rc}")
    res = {"out": out, "lse": lse}
    if lazy:
        res["lazy"] = lz
    if streaming:
        res["sout"], res["slse"] = so, sl
    return res


def decode(q, k_cache, v_cache, scale: Optional[float] = None, lib=None) -> Dict[str, np.ndarray]:
    """One decode query per (b, h): q [B,Hq,D]; caches [B,Hkv,L,D] (all L rows seen)."""
    q, k_cache, v_cache = _f64(q), _f64(k_cache), _f64(v_cache)
    B, Hq, D = q.shape
    _, Hkv, L, _ = k_cache.shape
    sc = default_scale(D) if scale is None else float(scale)
    out = np.empty((B, Hq, D)); lse = np.empty((B, Hq))
    rc = (lib or _load()).lto_decode(B, Hq, Hkv, D, sc, _ptr(q), _ptr(k_cache), _ptr(v_cache), L,
                            _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"lto_decode failed with code {rc}")
    return {"out": out, "lse": lse}


def prefill_varlen(q, k, v, seq_lens: Sequence[int], S: int = 0, R: int = 1, W: int = 0,
                   scale: Optional[float] = None, streaming: bool = False, full: bool = True,
                   lib=None) -> Dict[str, np.ndarray]:
    """A padded batch of sequences of different lengths: sequence b is its
    first seq_lens[b] positions, and the method runs on it alone (nothing in
    the pages couples the sequences of a batch).  Same outputs as prefill()
    in the padded [B, H, N] layout; entries at or past a sequence's length are
    NaN (no value).  Lazy ratio: each sequence observes its last
    min(W, seq_lens[b]) queries; lazy_rows[b, h, k] is row seq_lens[b] - W + k
    (NaN for rows before position 0) and lazy_ratio their mean (NaN for an
    empty sequence)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, N, D = q.shape
    res: Dict[str, np.ndarray] = {}
    if full:
        res["out"] = np.full((B, Hq, N, D), np.nan)
        res["lse"] = np.full((B, Hq, N), np.nan)
    if streaming:
        res["sout"] = np.full((B, Hq, N, D), np.nan)
        res["slse"] = np.full((B, Hq, N), np.nan)
    if W > 0:
        res["lazy_rows"] = np.full((B, Hq, W), np.nan)
        res["lazy_ratio"] = np.full((B, Hq), np.nan)
    for b in range(B):
        n = int(seq_lens[b])
        if not (0 <= n <= N):
            raise ValueError("sequence lengths must lie in [0, N]")
        if n == 0:
            continue
        w = min(W, n)
        one = prefill(q[b:b + 1, :, :n], k[b:b + 1, :, :n], v[b:b + 1, :, :n], S=S, R=R, W=w,
                      scale=scale, streaming=streaming, full=full, lib=lib)
        for key in ("out", "sout"):
            if key in one:
                res[key][b, :, :n] = one[key][0]
        for key in ("lse", "slse"):
            if key in one:
                res[key][b, :, :n] = one[key][0]
        if w > 0:
            res["lazy_rows"][b, :, W - w:] = one["lazy_rows"][0]
            res["lazy_ratio"][b] = one["lazy_ratio"][0]
    return res


def decode_varlen(q, k_cache, v_cache, kv_lens: Sequence[int], scale: Optional[float] = None,
                  lib=None) -> Dict[str, np.ndarray]:
    """Decode over caches of different lengths: sequence b attends to rows
    [0, kv_lens[b]) of its cache, alone.  An empty context has no softmax:
    out = 0 and lse = -inf (the conventions of an empty sum)."""
    q = _f64(q)
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(kv_lens[b])
        if n < 0 or n > k_cache.shape[2]:
            raise ValueError("kv_lens must lie in [0, rows]")
        if n == 0:
            continue
        one = decode(q[b:b + 1], _f64(k_cache[b:b + 1, :, :n]), _f64(v_cache[b:b + 1, :, :n]),
                     scale=scale, lib=lib)
        out[b], lse[b] = one["out"][0], one["lse"][0]
    return {"out": out, "lse": lse}



def gather_pages(pool, block_table, n: int, b: int):
    """Rows [0, n) of sequence b of a paged cache as one contiguous [Hkv, n, D]
    array: key j is row j % page_size of pool page block_table[b][j // page_size]
    (pool [num_pages, Hkv, page_size, D]); an entry outside [0, num_pages) is
    clamped into it, as the library's paged call documents."""
    pool = np.asarray(pool)
    num_pages, Hkv, P, D = pool.shape
    rows = np.empty((Hkv, n, D), dtype=np.float64)
    for j in range(n):
        pg = min(max(int(block_table[b][j // P]), 0), num_pages - 1)
        rows[:, j, :] = pool[pg, :, j % P, :]
    return rows


def decode_paged(q, k_pool, v_pool, block_table, kv_lens: Sequence[int], scale: Optional[float] = None,
                 lib=None) -> Dict[str, np.ndarray]:
    """Decode over paged caches: each sequence's keys gathered from the pools
    through the block table (gather_pages), then decode_varlen on them.  A
    length beyond max_pages * page_size is clamped to it; 0 gives out = 0,
    lse = -inf."""
    q = _f64(q)
    B, Hq, D = q.shape
    P = np.asarray(k_pool).shape[2]
    cap = len(block_table[0]) * P
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = min(max(int(kv_lens[b]), 0), cap)
        if n == 0:
            continue
        k = gather_pages(k_pool, block_table, n, b)[None]
        v = gather_pages(v_pool, block_table, n, b)[None]
        one = decode(q[b:b + 1], k, v, scale=scale, lib=lib)
        out[b], lse[b] = one["out"][0], one["lse"][0]
    return {"out": out, "lse": lse}

# ---------------------------------------------------------------------------
# Host-side selection (pure Python; small inputs by nature: one entry per layer)
# ---------------------------------------------------------------------------

def layer_score(head_ratio_row: Sequence[float]) -> float:
    """A layer's score: the mean of its per-(batch, head) lazy ratios, summed in
    fp64 in row-major order (the pages decide per layer and never mention heads)."""
    acc = 0.0
    for x in head_ratio_row:
        acc += float(x)
    return acc / len(head_ratio_row)


def select_lazy_layers(scores: Sequence[float], capacity: int,
                       policy: str = "after") -> Tuple[List[int], List[int]]:
    """Priority queue keyed by lazy ratio, updated after each layer
    (LightTransfer project page, Figure 2 caption; Chinese write-up,
    solution 2).

    policy "after" (the write-up's timing: a layer leaves once more layers
    are queued than the threshold): layer l is pushed as (score, l); while the
    queue holds more than ``capacity`` layers, the highest score leaves (equal
    scores: lower layer index first) and becomes a streaming layer.  policy
    "before" (the project page's timing: once the queue is full, the laziest
    layer leaves to make room for the current one): when ``capacity`` layers
    are already queued, the highest of them leaves first, then layer l is
    pushed; with capacity 0 every layer leaves at its own step.  Returns (evicted_at_step [L] with -1 for none,
    is_streaming [L] as 0/1)."""
    L = len(scores)
    if not (0 <= capacity <= L):
        raise ValueError("capacity must lie in [0, L]")
    if policy not in ("after", "before"):
        raise ValueError("policy must be 'after' or 'before'")
    heap: List[Tuple[float, int]] = []
    evicted = [-1] * L
    streaming = [0] * L
    for l, s in enumerate(scores):
        s = float(s)
        if math.isnan(s) or math.isinf(s):
            raise ValueError("scores must be finite")
        if policy == "before":
            if capacity == 0:
                victim = l
            else:
                victim = heapq.heappop(heap)[1] if len(heap) == capacity else -1
                heapq.heappush(heap, (-s, l))
        else:
            heapq.heappush(heap, (-s, l))
            victim = heapq.heappop(heap)[1] if len(heap) > capacity else -1
        if victim >= 0:
            evicted[l] = victim
            streaming[victim] = 1
    return evicted, streaming


def select_offline(prompt_scores: Sequence[Sequence[float]],
                   capacity: int) -> Tuple[List[float], List[int]]:
    """Offline lazy-layer selection (press-release page, "LightTransfer
    method", steps 1-3): measure every layer's lazy ratio on a set of prompts,
    call the layers with the highest ratios redundant and make them streaming
    layers.  The page fixes the share (50%) but not how the prompts are
    combined; here a layer's score is the mean of its per-prompt scores,
    summed in fp64 in prompt order.  ``capacity`` layers stay full: the
    L - capacity highest scores become streaming (equal scores: the lower
    layer index first, as in the queue).  Returns (mean score [L],
    is_streaming [L] as 0/1)."""
    P = len(prompt_scores)
    if P < 1:
        raise ValueError("need at least one prompt")
    L = len(prompt_scores[0])
    if L < 1 or any(len(row) != L for row in prompt_scores):
        raise ValueError("every prompt needs one score per layer")
    if not (0 <= capacity <= L):
        raise ValueError("capacity must lie in [0, L]")
    mean = []
    for l in range(L):
        acc = 0.0
        for p in range(P):
            x = float(prompt_scores[p][l])
            if math.isnan(x) or math.isinf(x):
                raise ValueError("scores must be finite")
            acc += x
        mean.append(acc / P)
    order = sorted(range(L), key=lambda l: (-mean[l], l))
    streaming = [0] * L
    for l in order[:L - capacity]:
        streaming[l] = 1
    return mean, streaming


def stream_slot(p: int, S: int, R: int) -> int:
    """Slot of position p in a streaming cache of S + R slots: the sinks keep
    their place, the recent positions go round a ring of R slots.  (The pages
    are silent on slot order; attention does not depend on it, and this order
    lets later tokens be appended in place.)"""
    return p if p < S else S + (p - S) % R


def streaming_rows(N: int, S: int, R: int) -> List[int]:
    """Positions a streaming KV cache of N tokens keeps, listed by slot: the
    sinks [0, S) and the recent [N-R, N) (the sink + recent set of the last
    query, N-1), position p in slot stream_slot(p); every row, in order, when
    N <= S + R."""
    if N <= S + R:
        return list(range(N))
    rows = [-1] * (S + R)
    for p in list(range(S)) + list(range(N - R, N)):
        rows[stream_slot(p, S, R)] = p
    return rows


def stream_append(rows: List[int], pos: int, S: int, R: int) -> List[int]:
    """The positions of a streaming cache (listed by slot, -1 = empty) after
    the token at position pos is written to its slot."""
    out = list(rows) + [-1] * max(0, S + R - len(rows))
    out[stream_slot(pos, S, R)] = pos
    return out


def kv_bytes(B: int, Hkv: int, N: int, D: int, elem: int, S: int, R: int) -> Tuple[int, int]:
    """(full, streaming) KV bytes of one layer: K and V, B*Hkv heads, D each."""
    full = 2 * B * Hkv * N * D * elem
    stream = 2 * B * Hkv * min(N, S + R) * D * elem
    return full, stream


def kv_accounting(evicted_at_step: Sequence[int], full: int, stream: int,
                  policy: str = "after", emit: bool = False) -> Dict[str, List[int]]:
    """Per-step KV bytes while prefill walks the layers.

    transient[l]: every layer so far at its current size plus layer l at full
    size, before the queue's pop -- except that with eviction before the push
    a victim from an earlier layer is already streaming (its memory is freed
    for layer l).  retained[l]: the same after the pop.  With ``emit`` every
    layer's prefill also produced its streaming slice, so a layer still at
    full size holds full + stream bytes (and switching it keeps the slice)."""
    L = len(evicted_at_step)
    is_stream = [False] * L
    retained, transient = [], []
    for l in range(L):
        ev = evicted_at_step[l]
        if policy == "before" and 0 <= ev < l:
            is_stream[ev] = True
        at_full = full + stream if emit else full
        before = sum(stream if is_stream[x] else at_full for x in range(l)) + at_full
        if ev >= 0:
            is_stream[ev] = True
        after = sum(stream if is_stream[x] else at_full for x in range(l + 1))
        transient.append(before)
        retained.append(after)
    return {"transient": transient, "retained": retained}
