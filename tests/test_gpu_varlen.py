"""GPU parity of the variable-length (padded) batch calls against the oracle.

Every sequence of a batch has its own length, read by the kernels from a
device array.  Padding rows hold large values, so a kernel that read them
would miss the oracle by far; output rows past a sequence's end are filled
with a sentinel beforehand and must keep it.  Lengths cover 0, 1, ragged
tiles, shorter than the observation window W, and the full padded size.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_causal_amd import api, ops, synth
from helpers import TOL_BF16_LSE, TOL_BF16_OUT, TOL_BF16_RATIO, TOL_F32, assert_close, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENT_OUT, SENT_LSE = 3.0, 5.0


def _tol(dtype):
    if dtype == torch.float32:
        return TOL_F32, TOL_F32, TOL_F32
    return TOL_BF16_OUT, TOL_BF16_LSE, TOL_BF16_RATIO


def _padded_qkv(lens, N, Hq, Hkv, D, dtype, seed):
    q, k, v = synth.qkv(len(lens), N, Hq, Hkv, D, seed, dtype)
    for b, n in enumerate(lens):
        q[b, :, n:] = 40.0
        k[b, :, n:] = 40.0
        v[b, :, n:] = -300.0
    return q, k, v


PREFILL_CASES = [
    # N, Hq, Hkv, D, dtype, S, R, W, lens, seed
    (300, 10, 2, 128, torch.bfloat16, 4, 60, 32, [300, 1, 77, 0, 250], 31),   # G=5
    (257, 4, 2, 64, torch.bfloat16, 4, 33, 16, [257, 200, 15, 16], 32),       # G=2, D=64
    (400, 16, 2, 128, torch.bfloat16, 4, 100, 40, [400, 399, 385, 1], 33),    # G=8
    (333, 3, 3, 128, torch.bfloat16, 0, 50, 20, [333, 129, 128], 34),         # G=1, S=0
    (200, 8, 2, 128, torch.float32, 4, 60, 50, [200, 3, 120], 35),            # fp32
    (130, 6, 3, 64, torch.float32, 0, 7, 130, [130, 1, 64, 0], 36),           # fp32, W=N
    # long windows: unmasked steps inside every row's window, skipped steps below it
    (800, 8, 2, 128, torch.bfloat16, 4, 250, 32, [800, 640, 300, 33], 37),    # G=4
    (700, 5, 1, 64, torch.bfloat16, 40, 180, 24, [700, 500, 41], 38),         # G=5, D=64, a step of sinks only
    (2500, 4, 2, 64, torch.bfloat16, 4, 100, 2100, [2500, 1500, 1030], 39),  # W > 1024, shorter sequences than W
]


@pytest.mark.parametrize("N,Hq,Hkv,D,dtype,S,R,W,lens,seed", PREFILL_CASES)
def test_prefill_varlen(N, Hq, Hkv, D, dtype, S, R, W, lens, seed):
    print(f"varlen prefill N{N} Hq{Hq} Hkv{Hkv} D{D} {dtype} S{S} R{R} W{W} lens {lens}", flush=True)
    B = len(lens)
    q, k, v = _padded_qkv(lens, N, Hq, Hkv, D, dtype, seed)
    ref = oracle.prefill_varlen(np64(q), np64(k), np64(v), lens, S=S, R=R, W=W, streaming=True)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lens_d = torch.tensor(lens, device=DEV, dtype=torch.int32)
    out = torch.full_like(qd, SENT_OUT)
    lse = torch.full((B, Hq, N), SENT_LSE, device=DEV, dtype=torch.float32)
    rows = torch.full((B, Hq, W), SENT_LSE, device=DEV, dtype=torch.float32)
    ratio = torch.full((B, Hq), SENT_LSE, device=DEV, dtype=torch.float32)
    api.lt_prefill_attn_lse_lazy_varlen(qd, kd, vd, out, lse, lens_d, S, R, W, rows, ratio)
    sout = torch.full_like(qd, SENT_OUT)
    slse = torch.full((B, Hq, N), SENT_LSE, device=DEV, dtype=torch.float32)
    api.lt_streaming_attn_varlen(qd, kd, vd, sout, slse, lens_d, S, R)
    torch.cuda.synchronize()
    to, tl, tr = _tol(dtype)
    got_rows, got_ratio = np64(rows), np64(ratio)
    for b, n in enumerate(lens):
        assert_close(f"out b{b}", np64(out[b, :, :n]), ref["out"][b, :, :n], to)
        assert_close(f"lse b{b}", np64(lse[b, :, :n]), ref["lse"][b, :, :n], tl)
        assert_close(f"stream out b{b}", np64(sout[b, :, :n]), ref["sout"][b, :, :n], to)
        assert_close(f"stream lse b{b}", np64(slse[b, :, :n]), ref["slse"][b, :, :n], tl)
        assert (np64(out[b, :, n:]) == SENT_OUT).all() and (np64(sout[b, :, n:]) == SENT_OUT).all()
        assert (np64(lse[b, :, n:]) == SENT_LSE).all() and (np64(slse[b, :, n:]) == SENT_LSE).all()
        w = min(W, n)
        assert_close(f"lazy rows b{b}", got_rows[b, :, W - w:], ref["lazy_rows"][b, :, W - w:], tr)
        assert np.isnan(got_rows[b, :, :W - w]).all()
        if n == 0:
            assert np.isnan(got_ratio[b]).all()
        else:
            assert_close(f"lazy ratio b{b}", got_ratio[b], ref["lazy_ratio"][b], tr)


@pytest.mark.parametrize("N,Hq,Hkv,D,dtype,S,R,W,lens,seed", PREFILL_CASES[:1] + PREFILL_CASES[4:5])
def test_prefill_varlen_full_lengths_equal_uniform_call(N, Hq, Hkv, D, dtype, S, R, W, lens, seed):
    """All lengths = N: the varlen call gives the uniform call's bits."""
    B = len(lens)
    q, k, v = (t.to(DEV) for t in synth.qkv(B, N, Hq, Hkv, D, seed, dtype))
    a = ops.prefill(q, k, v, S, R, W)
    b = ops.prefill_varlen(q, k, v, [N] * B, S, R, W)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


DECODE_CASES = [
    # Hq, Hkv, D, max_len, dtype, kv_lens, seed
    (10, 2, 128, 1000, torch.bfloat16, [1000, 1, 0, 523, 64], 41),
    (32, 2, 128, 5000, torch.bfloat16, [4999, 5000, 17, 2048], 42),   # G=16
    (8, 8, 64, 700, torch.bfloat16, [700, 63, 65, 0], 43),            # G=1, D=64
    (8, 2, 64, 900, torch.float32, [900, 1, 0, 450], 44),
    (4, 1, 128, 300, torch.float32, [300, 129, 2], 45),
    (40, 1, 128, 2000, torch.bfloat16, [2000, 0, 731, 1], 47),        # G=40: three chunks of query heads
    (10, 2, 64, 1200, torch.bfloat16, [(37 * i) % 1201 for i in range(33)], 48),  # B=33
]


@pytest.mark.parametrize("Hq,Hkv,D,L,dtype,lens,seed", DECODE_CASES)
def test_decode_varlen(Hq, Hkv, D, L, dtype, lens, seed):
    print(f"varlen decode Hq{Hq} Hkv{Hkv} D{D} L{L} {dtype} lens {lens}", flush=True)
    B = len(lens)
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, D, generator=g).to(dtype)
    k = torch.randn(B, Hkv, L, D, generator=g).to(dtype)
    v = torch.randn(B, Hkv, L, D, generator=g).to(dtype)
    for b, n in enumerate(lens):
        k[b, :, n:] = 40.0
        v[b, :, n:] = -300.0
    ref = oracle.decode_varlen(np64(q), np64(k), np64(v), lens)
    out, lse = ops.decode_varlen(q.to(DEV), k.to(DEV), v.to(DEV), lens, L)
    torch.cuda.synchronize()
    to, tl, _ = _tol(dtype)
    for b, n in enumerate(lens):
        if n == 0:
            assert (np64(out[b]) == 0).all() and (np64(lse[b]) == -np.inf).all()
            continue
        assert_close(f"decode out b{b}", np64(out[b]), ref["out"][b], to)
        assert_close(f"decode lse b{b}", np64(lse[b]), ref["lse"][b], tl)


def test_decode_varlen_full_lengths_agree_with_uniform_call():
    """All contexts at full length: the varlen call (equal parts of the
    batch) and the uniform call (per-sequence splits) sum in different
    pieces, so they agree to rounding, not bit for bit."""
    g = torch.Generator().manual_seed(46)
    q = torch.randn(3, 10, 128, generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn(3, 2, 3000, 128, generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn(3, 2, 3000, 128, generator=g).to(torch.bfloat16).to(DEV)
    a = ops.decode(q, k, v)
    b = ops.decode_varlen(q, k, v, [3000] * 3)
    torch.cuda.synchronize()
    assert_close("out", np64(b[0]), np64(a[0]), TOL_BF16_OUT)
    assert_close("lse", np64(b[1]), np64(a[1]), 1e-4)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_compaction_varlen_bit_exact(dtype):
    N, S, R, Hkv, D = 300, 4, 60, 2, 128
    lens = [300, 10, 0, 150, 64, 65]
    B = len(lens)
    g = torch.Generator().manual_seed(47)
    kf = torch.randn(B, Hkv, N, D, generator=g).to(dtype)
    vf = torch.randn(B, Hkv, N, D, generator=g).to(dtype)
    ks = torch.full((B, Hkv, S + R, D), SENT_OUT, dtype=dtype, device=DEV)
    vs = torch.full_like(ks, SENT_OUT)
    api.lt_compact_kv_streaming_varlen(kf.to(DEV), vf.to(DEV), ks, vs,
                                       torch.tensor(lens, device=DEV, dtype=torch.int32), S, R)
    torch.cuda.synchronize()
    ksh, vsh = ks.cpu(), vs.cpu()
    for b, n in enumerate(lens):
        keep = oracle.streaming_rows(n, S, R)
        assert torch.equal(ksh[b, :, :len(keep)], kf[b, :, keep])
        assert torch.equal(vsh[b, :, :len(keep)], vf[b, :, keep])
        assert (ksh[b, :, len(keep):] == SENT_OUT).all() and (vsh[b, :, len(keep):] == SENT_OUT).all()


def test_append_varlen_bit_exact():
    S, R, Hkv, D = 4, 60, 2, 128
    pos = [5, -1, 100, 0, 63, 64, 3]
    B = len(pos)
    g = torch.Generator().manual_seed(48)
    ks0 = torch.randn(B, Hkv, S + R, D, generator=g).to(torch.bfloat16)
    vs0 = torch.randn(B, Hkv, S + R, D, generator=g).to(torch.bfloat16)
    kn = torch.randn(B, Hkv, D, generator=g).to(torch.bfloat16)
    vn = torch.randn(B, Hkv, D, generator=g).to(torch.bfloat16)
    ks, vs = ks0.to(DEV), vs0.to(DEV)
    api.lt_stream_cache_append_varlen(ks, vs, kn.to(DEV), vn.to(DEV), S, R,
                                      torch.tensor(pos, device=DEV, dtype=torch.int32))
    torch.cuda.synchronize()
    want_k, want_v = ks0.clone(), vs0.clone()
    for b, p in enumerate(pos):
        if p >= 0:
            sl = oracle.stream_slot(p, S, R)
            want_k[b, :, sl] = kn[b]
            want_v[b, :, sl] = vn[b]
    assert torch.equal(ks.cpu(), want_k) and torch.equal(vs.cpu(), want_v)


def test_decode_varlen_graph_replay_with_new_lengths():
    """One captured HIP graph of the varlen decode, replayed after writing new
    lengths into the device array: every replay matches the oracle at its
    lengths (eager work and a synchronisation between replays)."""
    Hq, Hkv, D, L = 10, 2, 128, 3000
    B = 4
    g = torch.Generator().manual_seed(49)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hkv, L, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, L, D, generator=g).to(torch.bfloat16)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lens = torch.tensor([L] * B, device=DEV, dtype=torch.int32)
    ws = ops.decode_workspace(B, Hq, Hkv, D, L, DEV)
    out = torch.empty_like(qd)
    lse = torch.empty(B, Hq, device=DEV, dtype=torch.float32)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        api.lt_hybrid_decode_attn_varlen(qd, kd, vd, lens, L, out, lse, ws, 0.0, s)   # warm call
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        api.lt_hybrid_decode_attn_varlen(qd, kd, vd, lens, L, out, lse, ws, 0.0, s)
    torch.cuda.synchronize()
    for new in ([3000, 1, 1500, 0], [17, 2999, 64, 2048], [1, 1, 1, 3000]):
        lens.copy_(torch.tensor(new, dtype=torch.int32))       # eager, outside the graph
        _ = (qd.float() * 2.0).sum()                           # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle.decode_varlen(np64(q), np64(k), np64(v), new)
        for b, n in enumerate(new):
            if n == 0:
                assert (np64(out[b]) == 0).all() and (np64(lse[b]) == -np.inf).all()
                continue
            assert_close(f"replay {new} out b{b}", np64(out[b]), ref["out"][b], TOL_BF16_OUT)
            assert_close(f"replay {new} lse b{b}", np64(lse[b]), ref["lse"][b], TOL_BF16_LSE)
