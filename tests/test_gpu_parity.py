"""GPU parity: every kernel through the C ABI against the fp64 oracle.

Small shapes span several tiles and a ragged tail; GQA group sizes 1-8 cover
every workgroup layout; edge cases: N = 1, W = N, S = 0, S + R >= N.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_causal_amd import ops, synth
from helpers import (TOL_BF16_LSE, TOL_BF16_OUT, TOL_BF16_RATIO, TOL_F32, assert_close, np64)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _tol(dtype):
    if dtype == torch.float32:
        return TOL_F32, TOL_F32, TOL_F32
    return TOL_BF16_OUT, TOL_BF16_LSE, TOL_BF16_RATIO


PREFILL_CASES = [
    # B, N, Hq, Hkv, D, dtype, S, R, W, seed
    (1, 512, 4, 1, 64, torch.float32, 4, 60, 32, 1),      # tiny workload shape
    (1, 200, 8, 2, 128, torch.bfloat16, 4, 60, 32, 11),   # G=4, ragged
    (2, 300, 10, 2, 128, torch.bfloat16, 4, 100, 40, 12), # G=5, B=2
    (1, 333, 3, 3, 128, torch.bfloat16, 2, 50, 20, 13),   # G=1
    (1, 257, 4, 2, 64, torch.bfloat16, 4, 33, 16, 14),    # G=2, D=64
    (1, 190, 6, 2, 128, torch.bfloat16, 3, 70, 25, 15),   # G=3
    (1, 150, 16, 2, 128, torch.bfloat16, 4, 40, 30, 16),  # G=8 (two chunks)
    (1, 1, 5, 1, 128, torch.bfloat16, 4, 10, 1, 17),      # N=1
    (1, 17, 5, 1, 128, torch.bfloat16, 0, 5, 17, 18),     # S=0, W=N
    (1, 40, 5, 1, 128, torch.bfloat16, 8, 64, 10, 19),    # S+R >= N
    (1, 300, 8, 2, 128, torch.float32, 4, 60, 50, 20),    # fp32 D=128 G=4
    (2, 130, 6, 3, 64, torch.float32, 0, 7, 130, 21),     # fp32 W=N S=0
    (1, 150, 32, 2, 128, torch.bfloat16, 4, 40, 30, 22),  # G=16
    (1, 97, 16, 1, 64, torch.bfloat16, 4, 20, 9, 23),     # G=16, D=64
    (1, 2500, 4, 2, 64, torch.bfloat16, 4, 100, 2100, 24),  # W > 1024: the ratio's rows in several LDS rounds
    (1, 1100, 10, 2, 128, torch.bfloat16, 100, 300, 300, 25),  # sinks over two tiles, observed rows reach them
    (1, 900, 8, 1, 64, torch.bfloat16, 200, 64, 500, 26),      # sinks over two 128-key tiles
    (1, 2300, 10, 2, 128, torch.bfloat16, 1200, 2000, 300, 27),  # long sinks and window: S + R > N
]


@pytest.mark.parametrize("B,N,Hq,Hkv,D,dtype,S,R,W,seed", PREFILL_CASES)
def test_prefill_lse_lazy(B, N, Hq, Hkv, D, dtype, S, R, W, seed):
    print(f"prefill case B{B} N{N} Hq{Hq} Hkv{Hkv} D{D} {dtype} S{S} R{R} W{W}", flush=True)
    q, k, v = synth.qkv(B, N, Hq, Hkv, D, seed, dtype)
    ref = oracle.prefill(np64(q), np64(k), np64(v), S=S, R=R, W=W)
    out, lse, rows, ratio = ops.prefill(q.to(DEV), k.to(DEV), v.to(DEV), S, R, W)
    torch.cuda.synchronize()
    to, tl, tr = _tol(dtype)
    assert_close("out", np64(out), ref["out"], to)
    assert_close("lse", np64(lse), ref["lse"], tl)
    assert_close("lazy_rows", np64(rows), ref["lazy_rows"], tr)
    assert_close("lazy_ratio", np64(ratio), ref["lazy_ratio"], tr)


@pytest.mark.parametrize("D", [128, 64])
def test_prefill_large_grid_shape(D):
    """A grid of at least four 8-wave workgroups per CU (here 1024 on 256
    CUs) runs the 8-wave, 128-key shape (smaller grids, as in the cases
    above, take the 4-wave, 64-key one): out, LSE, the lazy rows and the
    ratio on sampled rows of every head against the oracle, a ragged tail
    included.  The streaming kernel on the same tensors too."""
    B, N, Hq, Hkv, S, R, W = 1, 6140, 64, 8, 4, 300, 48
    print(f"large-grid prefill D{D} B{B} N{N} Hq{Hq} Hkv{Hkv}", flush=True)
    q, k, v = synth.qkv(B, N, Hq, Hkv, D, 31 + D, torch.bfloat16, device=DEV)
    out, lse, rows, ratio = ops.prefill(q, k, v, S, R, W)
    sout, slse = ops.streaming(q, k, v, S, R)
    torch.cuda.synchronize()
    G = Hq // Hkv
    rng = np.random.default_rng(D)
    for h in range(Hq):
        pos = np.unique(np.concatenate([np.arange(N - W, N), np.arange(0, 8), rng.integers(0, N, 6)])).astype(np.int32)
        pt = torch.as_tensor(pos, device=DEV, dtype=torch.long)
        r = oracle.rows(np64(k[0, h // G]), np64(v[0, h // G]), pos, np64(q[0, h][pt]), S=S, R=R)
        assert_close(f"out h{h}", np64(out[0, h][pt]), r["out"], TOL_BF16_OUT)
        assert_close(f"lse h{h}", np64(lse[0, h][pt]), r["lse"], TOL_BF16_LSE)
        assert_close(f"stream out h{h}", np64(sout[0, h][pt]), r["sout"], TOL_BF16_OUT)
        assert_close(f"stream lse h{h}", np64(slse[0, h][pt]), r["slse"], TOL_BF16_LSE)
        obs = pos >= N - W
        assert_close(f"lazy rows h{h}", np64(rows[0, h]), r["lazy"][obs], TOL_BF16_RATIO)
        assert abs(float(ratio[0, h]) - r["lazy"][obs].mean()) <= TOL_BF16_RATIO


@pytest.mark.parametrize("B,N,Hq,Hkv,D,dtype,S,R,W,seed", PREFILL_CASES)
def test_prefill_plain_matches_lazy_variant(B, N, Hq, Hkv, D, dtype, S, R, W, seed):
    """W = 0 runs the kernel without the epilogue: out and lse are bit-identical."""
    q, k, v = (t.to(DEV) for t in synth.qkv(B, N, Hq, Hkv, D, seed, dtype))
    out0, lse0, _, _ = ops.prefill(q, k, v, S, R, 0)
    out1, lse1, _, _ = ops.prefill(q, k, v, S, R, W)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)


STREAM_CASES = [
    (1, 512, 4, 1, 64, torch.float32, 4, 60, 1),
    (1, 300, 8, 2, 128, torch.bfloat16, 4, 60, 2),
    (2, 333, 10, 2, 128, torch.bfloat16, 4, 100, 3),
    (1, 260, 3, 3, 128, torch.bfloat16, 0, 37, 4),
    (1, 200, 4, 2, 64, torch.bfloat16, 70, 1, 5),      # R = 1: sinks + diagonal
    (1, 100, 16, 2, 128, torch.bfloat16, 4, 200, 6),   # S + R >= N: full attention
    (1, 257, 6, 2, 128, torch.float32, 3, 64, 7),
    # long windows: steps wholly inside every row's window run unmasked, and
    # non-sink steps below every window are skipped
    (1, 900, 2, 2, 128, torch.bfloat16, 4, 300, 8),    # G=1
    (1, 700, 16, 2, 128, torch.bfloat16, 5, 250, 9),   # G=8
    (1, 640, 4, 2, 64, torch.bfloat16, 33, 150, 10),   # a step of sinks only, then a mixed one
    (1, 800, 5, 1, 128, torch.bfloat16, 64, 128, 11),  # two whole sink steps
    (1, 300, 32, 2, 128, torch.bfloat16, 4, 60, 12),   # G=16
    # sinks over two or three 64-key tiles, with windows that reach into them
    (1, 900, 10, 2, 128, torch.bfloat16, 100, 300, 13),
    (1, 1500, 8, 1, 64, torch.bfloat16, 130, 200, 14),
    (2, 700, 6, 3, 128, torch.float32, 150, 90, 15),
    # many sink tiles before the band, and sinks past the sequence's end
    (1, 2500, 8, 2, 128, torch.bfloat16, 1500, 37, 16),
    (1, 900, 5, 1, 64, torch.bfloat16, 905, 3, 17),
]


@pytest.mark.parametrize("B,N,Hq,Hkv,D,dtype,S,R,seed", STREAM_CASES)
def test_streaming(B, N, Hq, Hkv, D, dtype, S, R, seed):
    print(f"streaming case B{B} N{N} Hq{Hq} Hkv{Hkv} D{D} {dtype} S{S} R{R}", flush=True)
    q, k, v = synth.qkv(B, N, Hq, Hkv, D, seed, dtype)
    ref = oracle.prefill(np64(q), np64(k), np64(v), S=S, R=R, W=0, streaming=True, full=False)
    out, lse = ops.streaming(q.to(DEV), k.to(DEV), v.to(DEV), S, R)
    torch.cuda.synchronize()
    to, tl, _ = _tol(dtype)
    assert_close("sout", np64(out), ref["sout"], to)
    assert_close("slse", np64(lse), ref["slse"], tl)


DECODE_CASES = [
    # B, Hq, Hkv, D, L, dtype, seed
    (2, 10, 2, 128, 1, torch.bfloat16, 1),
    (2, 10, 2, 128, 100, torch.bfloat16, 2),
    (1, 40, 8, 128, 1024, torch.bfloat16, 3),
    (3, 8, 2, 64, 5000, torch.bfloat16, 4),
    (1, 16, 1, 128, 777, torch.bfloat16, 5),   # G = 16
    (2, 4, 4, 128, 3000, torch.bfloat16, 6),   # G = 1
    (2, 10, 2, 128, 700, torch.float32, 7),
    (1, 4, 1, 64, 65, torch.float32, 8),
    # more than 16 query heads per KV head: chunks of 16 columns
    (1, 40, 1, 128, 3000, torch.bfloat16, 9),    # G = 40, multi-query
    (2, 64, 2, 64, 777, torch.bfloat16, 10),     # G = 32
    (3, 20, 1, 128, 100, torch.bfloat16, 11),    # G = 20
    (1, 48, 2, 128, 500, torch.float32, 12),     # G = 24, fp32
    (64, 16, 2, 128, 300, torch.bfloat16, 13),   # large batch: one split per (sequence, KV head)
]


@pytest.mark.parametrize("B,Hq,Hkv,D,L,dtype,seed", DECODE_CASES)
def test_decode(B, Hq, Hkv, D, L, dtype, seed):
    print(f"decode case B{B} Hq{Hq} Hkv{Hkv} D{D} L{L} {dtype}", flush=True)
    q = synth.normal((B, Hq, D), seed, dtype)
    k = synth.normal((B, Hkv, L, D), seed + 100, dtype)
    v = synth.normal((B, Hkv, L, D), seed + 200, dtype)
    ref = oracle.decode(np64(q), np64(k), np64(v))
    out, lse = ops.decode(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    to, tl, _ = _tol(dtype)
    assert_close("out", np64(out), ref["out"], to)
    assert_close("lse", np64(lse), ref["lse"], tl)


@pytest.mark.parametrize("N,S,R,dtype", [(300, 4, 60, torch.bfloat16), (50, 4, 60, torch.bfloat16),
                                         (1000, 0, 100, torch.float32), (64, 64, 1, torch.bfloat16)])
def test_compaction_bit_exact(N, S, R, dtype):
    k = synth.normal((2, 3, N, 128), 31, dtype)
    v = synth.normal((2, 3, N, 128), 32, dtype)
    ks, vs = ops.compact(k.to(DEV), v.to(DEV), S, R)
    torch.cuda.synchronize()
    idx = oracle.streaming_rows(N, S, R)
    assert torch.equal(ks.cpu(), k[:, :, idx, :])
    assert torch.equal(vs.cpu(), v[:, :, idx, :])


@pytest.mark.parametrize("N0,T,S,R,dtype", [(300, 70, 4, 60, torch.bfloat16), (20, 50, 4, 30, torch.bfloat16),
                                            (100, 40, 0, 16, torch.float32)])
def test_streaming_decode_with_appends(N0, T, S, R, dtype):
    """Prefill a layer of N0 tokens, compact it to a streaming cache of S+R
    slots, then decode T more tokens, appending each one first: every step
    equals the oracle's streaming attention of that token over the whole
    sequence (sink + recent keys)."""
    from kv_cache_compression_causal_amd import api
    print(f"streaming decode with appends N0={N0} T={T} S={S} R={R} {dtype}", flush=True)
    B, Hq, Hkv, D = 2, 10, 2, 128
    N = N0 + T
    q, k, v = synth.qkv(B, N, Hq, Hkv, D, 91, dtype)
    ref = oracle.prefill(np64(q), np64(k), np64(v), S=S, R=R, streaming=True, full=False)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ks, vs = ops.compact(kd[:, :, :N0].contiguous(), vd[:, :, :N0].contiguous(), S, R, slots=S + R)
    ws = ops.decode_workspace(B, Hq, Hkv, D, S + R, DEV)
    to, tl, _ = _tol(dtype)
    for pos in range(N0, N):
        kv_len = ops.stream_append(ks, vs, kd[:, :, pos], vd[:, :, pos], S, R, pos)
        out = torch.empty(B, Hq, D, device=DEV, dtype=dtype)
        lse = torch.empty(B, Hq, device=DEV, dtype=torch.float32)
        api.lt_hybrid_decode_attn(qd[:, :, pos].contiguous(), ks, vs, kv_len, out, lse, ws)
        torch.cuda.synchronize()
        assert_close(f"out@{pos}", np64(out), ref["sout"][:, :, pos], to)
        assert_close(f"lse@{pos}", np64(lse), ref["slse"][:, :, pos], tl)


def test_lazy_ratio_equals_streaming_lse_gap():
    """Per-row lazy ratio = exp(LSE_stream - LSE_full): two kernels, one identity."""
    B, N, Hq, Hkv, D, S, R, W = 1, 700, 10, 2, 128, 4, 100, 64
    q, k, v = (t.to(DEV) for t in synth.qkv(B, N, Hq, Hkv, D, 41, torch.bfloat16))
    _, lse, rows, _ = ops.prefill(q, k, v, S, R, W)
    _, slse = ops.streaming(q, k, v, S, R)
    torch.cuda.synchronize()
    gap = torch.exp((slse[:, :, N - W:] - lse[:, :, N - W:]).double())
    assert_close("ratio vs lse gap", np64(rows), gap.cpu().numpy(), 2e-3)


def test_decode_on_compacted_cache_matches_streaming_last_row():
    """Streaming decode over the compacted cache = streaming prefill at row N-1."""
    B, N, Hq, Hkv, D, S, R = 2, 600, 10, 2, 128, 4, 100
    q, k, v = (t.to(DEV) for t in synth.qkv(B, N, Hq, Hkv, D, 42, torch.bfloat16))
    sout, slse = ops.streaming(q, k, v, S, R)
    ks, vs = ops.compact(k, v, S, R)
    dout, dlse = ops.decode(q[:, :, N - 1, :].contiguous(), ks, vs)
    torch.cuda.synchronize()
    assert_close("out", np64(dout), np64(sout[:, :, N - 1, :]), 2e-2)
    assert_close("lse", np64(dlse), np64(slse[:, :, N - 1]), 1e-3)


def test_deterministic():
    q, k, v = (t.to(DEV) for t in synth.qkv(1, 500, 10, 2, 128, 43, torch.bfloat16))
    a = ops.prefill(q, k, v, 4, 60, 50)
    b = ops.prefill(q, k, v, 4, 60, 50)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


EMIT_CASES = [
    # B, N, Hq, Hkv, D, dtype, S, R, W, lens (None: every sequence N rows), seed
    (1, 300, 10, 2, 128, torch.bfloat16, 4, 60, 32, None, 51),     # ring order, G=5
    (2, 50, 8, 2, 128, torch.bfloat16, 4, 60, 16, None, 52),       # N <= S+R: every row, in order
    (1, 333, 3, 3, 64, torch.bfloat16, 0, 37, 20, None, 53),       # S=0, G=1, D=64
    (1, 400, 16, 2, 128, torch.bfloat16, 4, 100, 40, None, 54),    # G=8
    (1, 200, 8, 2, 128, torch.float32, 4, 60, 50, None, 55),       # fp32
    (4, 300, 10, 2, 128, torch.bfloat16, 4, 60, 32, [300, 1, 64, 0], 56),  # varlen: short, empty
    (3, 130, 6, 3, 64, torch.float32, 2, 30, 10, [130, 33, 31], 57),       # fp32 varlen
]


@pytest.mark.parametrize("B,N,Hq,Hkv,D,dtype,S,R,W,lens,seed", EMIT_CASES)
def test_prefill_emits_streaming_slice(B, N, Hq, Hkv, D, dtype, S, R, W, lens, seed):
    """The prefill that writes the streaming slice: the slice equals the
    oracle's row set in ring slot order bit for bit (slots past it keep a
    sentinel), and the attention outputs are those of the call without it."""
    print(f"emit case B{B} N{N} Hq{Hq} Hkv{Hkv} D{D} {dtype} S{S} R{R} W{W} lens {lens}", flush=True)
    q, k, v = (t.to(DEV) for t in synth.qkv(B, N, Hq, Hkv, D, seed, dtype))
    n_of = [N] * B if lens is None else lens
    lens_d = None if lens is None else torch.tensor(lens, device=DEV, dtype=torch.int32)
    if lens is None:
        ref = ops.prefill(q, k, v, S, R, W)
    else:
        ref = ops.prefill_varlen(q, k, v, lens, S, R, W)
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, N, device=DEV, dtype=torch.float32)
    rows = torch.empty(B, Hq, W, device=DEV, dtype=torch.float32)
    ratio = torch.empty(B, Hq, device=DEV, dtype=torch.float32)
    ks = torch.full((B, Hkv, S + R, D), 7.0, device=DEV, dtype=dtype)
    vs = torch.full_like(ks, 7.0)
    from kv_cache_compression_causal_amd import api
    api.lt_prefill_attn_lse_lazy_emit(q, k, v, out, lse, S, R, W, rows, ratio, ks, vs, lens_d)
    torch.cuda.synchronize()
    kh, vh, ksh, vsh = k.cpu(), v.cpu(), ks.cpu(), vs.cpu()
    for b, n in enumerate(n_of):
        assert torch.equal(out[b, :, :n], ref[0][b, :, :n]) and torch.equal(lse[b, :, :n], ref[1][b, :, :n])
        assert torch.allclose(rows[b], ref[2][b], rtol=0, atol=0, equal_nan=True)
        assert torch.allclose(ratio[b], ref[3][b], rtol=0, atol=0, equal_nan=True)
        keep = oracle.streaming_rows(n, S, R)
        assert torch.equal(ksh[b, :, :len(keep)], kh[b, :, keep]) and torch.equal(vsh[b, :, :len(keep)], vh[b, :, keep])
        assert (ksh[b, :, len(keep):] == 7.0).all() and (vsh[b, :, len(keep):] == 7.0).all()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_permuted_views_match_contiguous(dtype):
    """Tensors stored as [B, N, H, D] (row stride H*D, head stride D) and passed
    as permuted [B, H, N, D] views: prefill + lazy, streaming, the emitted
    slice, compaction and decode give the contiguous calls' bits (the same
    arithmetic at other addresses; the contiguous results are checked
    against the oracle elsewhere)."""
    from kv_cache_compression_causal_amd import api
    B, N, Hq, Hkv, D, S, R, W = 2, 300, 10, 2, 128, 4, 60, 32
    print(f"permuted views {dtype}", flush=True)
    q, k, v = (t.to(DEV) for t in synth.qkv(B, N, Hq, Hkv, D, 61, dtype))
    qp = q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)   # storage [B, N, Hq, D]
    kp = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    vp = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert qp.stride(2) == Hq * D and qp.stride(1) == D and qp.shape == q.shape
    ref = ops.prefill(q, k, v, S, R, W)
    out_p = torch.empty(B, N, Hq, D, device=DEV, dtype=dtype).permute(0, 2, 1, 3)
    lse = torch.empty(B, Hq, N, device=DEV, dtype=torch.float32)
    rows = torch.empty(B, Hq, W, device=DEV, dtype=torch.float32)
    ratio = torch.empty(B, Hq, device=DEV, dtype=torch.float32)
    ks_p = torch.empty(B, S + R, Hkv, D, device=DEV, dtype=dtype).permute(0, 2, 1, 3)
    vs_p = torch.empty_like(ks_p.permute(0, 2, 1, 3)).permute(0, 2, 1, 3)
    api.lt_prefill_attn_lse_lazy_emit(qp, kp, vp, out_p, lse, S, R, W, rows, ratio, ks_p, vs_p)
    sref = ops.streaming(q, k, v, S, R)
    sout_p = torch.empty(B, N, Hq, D, device=DEV, dtype=dtype).permute(0, 2, 1, 3)
    slse = torch.empty(B, Hq, N, device=DEV, dtype=torch.float32)
    api.lt_streaming_attn(qp, kp, vp, sout_p, slse, S, R)
    cks, cvs = ops.compact(k, v, S, R)
    cks_p = torch.empty(B, S + R, Hkv, D, device=DEV, dtype=dtype).permute(0, 2, 1, 3)
    cvs_p = torch.empty(B, S + R, Hkv, D, device=DEV, dtype=dtype).permute(0, 2, 1, 3)
    api.lt_compact_kv_streaming(kp, vp, cks_p, cvs_p, S, R)
    qd = q[:, :, N - 1].contiguous()
    dref = ops.decode(qd, k, v)
    dout = torch.empty_like(qd)
    dlse = torch.empty(B, Hq, device=DEV, dtype=torch.float32)
    api.lt_hybrid_decode_attn(qd, kp, vp, N, dout, dlse, ops.decode_workspace(B, Hq, Hkv, D, N, DEV))
    torch.cuda.synchronize()
    assert torch.equal(out_p, ref[0]) and torch.equal(lse, ref[1])
    assert torch.equal(rows, ref[2]) and torch.equal(ratio, ref[3])
    assert torch.equal(sout_p, sref[0]) and torch.equal(slse, sref[1])
    assert torch.equal(ks_p, cks) and torch.equal(vs_p, cvs)
    assert torch.equal(cks_p, cks) and torch.equal(cvs_p, cvs)
    assert torch.equal(dout, dref[0]) and torch.equal(dlse, dref[1])
    # the same views through the per-sequence-length calls
    lens = [N, N // 3]
    vref = ops.prefill_varlen(q, k, v, lens, S, R, W)
    vout_p = torch.empty(B, N, Hq, D, device=DEV, dtype=dtype).permute(0, 2, 1, 3)
    vlse = torch.empty(B, Hq, N, device=DEV, dtype=torch.float32)
    vrows = torch.empty(B, Hq, W, device=DEV, dtype=torch.float32)
    vratio = torch.empty(B, Hq, device=DEV, dtype=torch.float32)
    lens_d = torch.tensor(lens, device=DEV, dtype=torch.int32)
    api.lt_prefill_attn_lse_lazy_varlen(qp, kp, vp, vout_p, vlse, lens_d, S, R, W, vrows, vratio)
    kvref = ops.decode_varlen(qd, k, v, lens)
    kvout = torch.empty_like(qd)
    kvlse = torch.empty(B, Hq, device=DEV, dtype=torch.float32)
    api.lt_hybrid_decode_attn_varlen(qd, kp, vp, lens_d, N, kvout, kvlse,
                                     ops.decode_workspace(B, Hq, Hkv, D, N, DEV))
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        assert torch.equal(vout_p[b, :, :n], vref[0][b, :, :n]) and torch.equal(vlse[b, :, :n], vref[1][b, :, :n])
    assert torch.equal(vratio, vref[3]) and torch.equal(kvout, kvref[0]) and torch.equal(kvlse, kvref[1])


def test_debug_build_with_poisoned_lds_gives_the_same_bits():
    """liblt_debug.so (every kernel fills its LDS with NaN before first use)
    against liblt.so on the same inputs: identical bits for prefill + lazy
    (both workgroup shapes), fp32, streaming, the emitted slice and decode
    (uniform and per-sequence contexts), so no kernel reads LDS it did not
    write."""
    import contextlib
    from kv_cache_compression_causal_amd import _lib
    debug = _lib.load_library(_lib.DEBUG_LIB_PATH)
    release = _lib.lib()

    @contextlib.contextmanager
    def using(library):
        saved = _lib._lib
        _lib._lib = library
        try:
            yield
        finally:
            _lib._lib = saved

    def run():
        res = []
        for (B, N, Hq, Hkv, D, dtype, S, R, W, seed) in [(2, 300, 10, 2, 128, torch.bfloat16, 4, 100, 40, 41),
                                                         (1, 6140, 64, 8, 128, torch.bfloat16, 4, 300, 48, 42),
                                                         (1, 257, 4, 2, 64, torch.bfloat16, 4, 33, 16, 43),
                                                         (1, 300, 8, 2, 128, torch.float32, 4, 60, 50, 44)]:
            q, k, v = synth.qkv(B, N, Hq, Hkv, D, seed, dtype, device=DEV)
            res += list(ops.prefill(q, k, v, S, R, W)) + list(ops.streaming(q, k, v, S, R))
            res += list(ops.prefill_emit(q, k, v, S, R, W))
            qd = q[:, :, -1].contiguous()
            res += list(ops.decode(qd, k, v)) + list(ops.decode_varlen(qd, k, v, [N - 7 * b for b in range(B)]))
        torch.cuda.synchronize()
        return res

    print("release vs debug (LDS poisoned) library", flush=True)
    with using(release):
        want = run()
    with using(debug):
        got = run()
    assert len(got) == len(want)
    for i, (g_, w_) in enumerate(zip(got, want)):
        assert torch.equal(g_.view(torch.uint8), w_.view(torch.uint8)), f"output {i} differs"


def test_lt_log_prints_each_launch():
    """LT_LOG=1 on the GPU: the call line and the launch line naming the
    kernel and its grid (a child process, so the setting stays local)."""
    import os
    import subprocess
    import sys
    code = ("import torch\n"
            "from kv_cache_compression_causal_amd import ops, synth\n"
            "q, k, v = synth.qkv(1, 200, 8, 2, 128, 5, torch.bfloat16, device='cuda')\n"
            "ops.prefill(q, k, v, 4, 60, 32)\n"
            "torch.cuda.synchronize()\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=dict(os.environ, LT_LOG="1"),
                       capture_output=True, text=True, timeout=150)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "lt_prefill_attn_lse_lazy(B=1 N=200 Hq=8 Hkv=2 D=128" in r.stderr and "-> LT_OK" in r.stderr
    assert "launch attn_bf16_kernel<D=128" in r.stderr and "launch lazy_reduce_kernel" in r.stderr


def test_layer_calls_captured_in_a_graph():
    """Prefill + lazy ratio, streaming, compaction and decode of one layer
    (and a paged decode over the layer's K/V read as 32-row pages)
    captured in one HIP graph on a side stream, replayed three times after
    new inputs, a new page table and a new length were copied in eagerly
    (with unrelated eager work and a synchronisation between replays):
    every replay gives the eager calls' bits on the same inputs.  The
    library issues no memset or allocation, so nothing in the graph depends
    on capture-time state."""
    from kv_cache_compression_causal_amd import api
    B, N, Hq, Hkv, D, S, R, W = 1, 700, 8, 2, 128, 4, 100, 40
    G = Hq // Hkv
    q, k, v = (t.to(DEV) for t in synth.qkv(B, N, Hq, Hkv, D, 61, torch.bfloat16))
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, N, device=DEV, dtype=torch.float32)
    rows = torch.empty(B, Hq, W, device=DEV, dtype=torch.float32)
    ratio = torch.empty(B, Hq, device=DEV, dtype=torch.float32)
    sout = torch.empty_like(q)
    slse = torch.empty(B, Hq, N, device=DEV, dtype=torch.float32)
    ks = torch.empty(B, Hkv, S + R, D, device=DEV, dtype=torch.bfloat16)
    vs = torch.empty_like(ks)
    qt = torch.empty(B, Hq, D, device=DEV, dtype=torch.bfloat16)
    dout = torch.empty_like(qt)
    dlse = torch.empty(B, Hq, device=DEV, dtype=torch.float32)
    ws = ops.decode_workspace(B, Hq, Hkv, D, S + R, DEV)
    P, npg = 32, N // 32                                       # k, v [1, Hkv, N, D] as a pool of 32-row pages
    kp = torch.as_strided(k, (npg, Hkv, P, D), (P * D, N * D, D, 1))
    vp = torch.as_strided(v, (npg, Hkv, P, D), (P * D, N * D, D, 1))
    table = torch.as_tensor(np.random.default_rng(65).permutation(npg)[None], dtype=torch.int32).to(DEV)
    plens = torch.tensor([npg * P - 5], device=DEV, dtype=torch.int32)
    pws = ops.decode_workspace(B, Hq, Hkv, D, npg * P, DEV)
    pout = torch.empty_like(qt)
    plse = torch.empty(B, Hq, device=DEV, dtype=torch.float32)
    outs = (out, lse, rows, ratio, sout, slse, ks, vs, dout, dlse, pout, plse)

    def layer(st):
        api.lt_prefill_attn_lse_lazy(q, k, v, out, lse, S, R, W, rows, ratio, 0.0, st)
        api.lt_streaming_attn(q, k, v, sout, slse, S, R, 0.0, st)
        api.lt_compact_kv_streaming(k, v, ks, vs, S, R, st)
        qt.copy_(q[:, :, -1])
        api.lt_hybrid_decode_attn(qt, ks, vs, S + R, dout, dlse, ws, 0.0, st)
        api.lt_hybrid_decode_attn_paged(qt, kp, vp, table, plens, pout, plse, pws, 0.0, st)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer(s)                                              # warm call
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        layer(s)
    torch.cuda.synchronize()
    for seed in (62, 63, 64):
        print(f"graph replay, inputs seed {seed}", flush=True)
        nq, nk, nv = synth.qkv(B, N, Hq, Hkv, D, seed, torch.bfloat16)
        q.copy_(nq), k.copy_(nk), v.copy_(nv)
        # a new page order and length for the paged decode (read through the
        # scalar cache: a stale entry would make the replay differ from eager)
        table.copy_(torch.as_tensor(np.random.default_rng(seed).permutation(npg)[None], dtype=torch.int32))
        plens.fill_(npg * P - seed % 7)
        _ = (q.float() * 2.0).sum()                           # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        with torch.cuda.stream(s):
            layer(s)                                          # eager, same inputs
        torch.cuda.synchronize()
        for i, (g_, w_) in enumerate(zip(got, outs)):
            assert torch.equal(g_.view(torch.uint8), w_.view(torch.uint8)), f"replay (seed {seed}) output {i} differs"
    # and the eager results are right
    ref = oracle.prefill(np64(q), np64(k), np64(v), S=S, R=R, W=W, streaming=True)
    assert_close("out", np64(out), ref["out"], TOL_BF16_OUT)
    assert_close("lazy_ratio", np64(ratio), ref["lazy_ratio"], TOL_BF16_RATIO)
    assert_close("sout", np64(sout), ref["sout"], TOL_BF16_OUT)
    pref = oracle.decode_paged(np64(qt), np64(kp), np64(vp), table.cpu().numpy(), [int(plens.item())])
    assert_close("paged out", np64(pout), pref["out"], TOL_BF16_OUT)
    assert_close("paged lse", np64(plse), pref["lse"], TOL_BF16_LSE)


def test_calls_on_two_streams_at_once():
    """Two layers' calls issued on two streams without synchronising in
    between (prefill + lazy ratio, streaming, decode on each): the results
    equal, bit for bit, those of the same calls run one after the other.  The
    library keeps no state between calls (the allocation-free decode's array
    aside, which these calls do not use)."""
    from kv_cache_compression_causal_amd import api
    B, N, Hq, Hkv, D, S, R, W = 1, 3000, 16, 4, 128, 4, 300, 40
    sets = []
    for seed in (71, 72):
        q, k, v = (t.to(DEV) for t in synth.qkv(B, N, Hq, Hkv, D, seed, torch.bfloat16))
        outs = dict(out=torch.empty_like(q), lse=torch.empty(B, Hq, N, device=DEV),
                    rows=torch.empty(B, Hq, W, device=DEV), ratio=torch.empty(B, Hq, device=DEV),
                    sout=torch.empty_like(q), slse=torch.empty(B, Hq, N, device=DEV),
                    dout=torch.empty(B, Hq, D, device=DEV, dtype=torch.bfloat16),
                    dlse=torch.empty(B, Hq, device=DEV),
                    ws=ops.decode_workspace(B, Hq, Hkv, D, N, DEV), qt=q[:, :, -1].contiguous())
        sets.append((q, k, v, outs))

    def layer(q, k, v, o, st):
        api.lt_prefill_attn_lse_lazy(q, k, v, o["out"], o["lse"], S, R, W, o["rows"], o["ratio"], 0.0, st)
        api.lt_streaming_attn(q, k, v, o["sout"], o["slse"], S, R, 0.0, st)
        api.lt_hybrid_decode_attn(o["qt"], k, v, N, o["dout"], o["dlse"], o["ws"], 0.0, st)

    keys = ("out", "lse", "rows", "ratio", "sout", "slse", "dout", "dlse")
    cur = torch.cuda.current_stream()
    for q, k, v, o in sets:          # one after the other
        layer(q, k, v, o, cur)
        torch.cuda.synchronize()
    want = [{kk: o[kk].clone() for kk in keys} for _, _, _, o in sets]
    for _, _, _, o in sets:
        for kk in keys:
            o[kk].fill_(float("nan"))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        print(f"two streams, round {rep}", flush=True)
        for (q, k, v, o), st in zip(sets, (s1, s2)):
            st.wait_stream(cur)
            layer(q, k, v, o, st)
        torch.cuda.synchronize()
        for i, (_, _, _, o) in enumerate(sets):
            for kk in keys:
                assert torch.equal(o[kk].view(torch.uint8), want[i][kk].view(torch.uint8)), f"set {i} {kk} differs"
