"""GPU parity on keys whose scores jump far above the running maximum.

On N(0,1) inputs a row's running max settles within its first steps, so the
kernels' rescale path (a step whose weights outgrow the lagging max: the
row max is taken across lanes, O, l and the lazy numerator are rescaled and
the step's weights redone, the scores recomputed from the staged K tile in
place) would run almost only on a wave's first step.  Here single keys are
scaled by 16 or 100 at positions spread over tiles and steps: at the start,
on tile and step boundaries, inside the diagonal step of nearby rows (the
masked recompute), between the sinks and the window, and inside the recent
window of the observed rows.  A factor of 100 makes the first try of a
step's weights overflow to inf before the rescale.  Every kernel is checked
against the fp64 oracle: both prefill workgroup shapes, D = 128 and 64, fp32,
streaming, per-sequence lengths and decode.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_causal_amd import api, ops, synth
from helpers import (TOL_BF16_LSE, TOL_BF16_OUT, TOL_BF16_RATIO, TOL_F32, assert_close, np64)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _tol(dtype):
    if dtype == torch.float32:
        return TOL_F32, TOL_F32, TOL_F32
    return TOL_BF16_OUT, TOL_BF16_LSE, TOL_BF16_RATIO


def _spikes(N, extra=()):
    """Positions spread over the sequence, alternating factors 16 and 100."""
    pos = sorted({p for p in (1, 37, 63, 64, 127, 128, 129, 300, 301, N // 2, N - 90, N - 31, N - 5, *extra)
                  if 0 <= p < N})
    return [(p, 16.0 if i % 2 == 0 else 100.0) for i, p in enumerate(pos)]


SMALL_CASES = [
    # B, N, Hq, Hkv, D, dtype, S, R, W, seed
    (1, 700, 8, 2, 128, torch.bfloat16, 4, 100, 40, 71),
    (2, 333, 10, 2, 128, torch.bfloat16, 4, 60, 33, 72),   # G=5
    (1, 600, 4, 2, 64, torch.bfloat16, 40, 150, 64, 73),   # D=64, spikes among the sinks
    (1, 400, 6, 3, 128, torch.bfloat16, 0, 37, 20, 74),    # S=0
    (1, 512, 4, 1, 64, torch.float32, 4, 60, 32, 75),      # the fp32 kernel
    (1, 300, 8, 2, 128, torch.float32, 4, 60, 50, 76),
]


@pytest.mark.parametrize("B,N,Hq,Hkv,D,dtype,S,R,W,seed", SMALL_CASES)
def test_prefill_and_streaming_with_score_spikes(B, N, Hq, Hkv, D, dtype, S, R, W, seed):
    print(f"spiky prefill B{B} N{N} Hq{Hq} Hkv{Hkv} D{D} {dtype} S{S} R{R} W{W}", flush=True)
    q, k, v = synth.qkv(B, N, Hq, Hkv, D, seed, dtype, spikes=_spikes(N, (S - 1, S, S + 1)))
    ref = oracle.prefill(np64(q), np64(k), np64(v), S=S, R=R, W=W, streaming=True)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse, rows, ratio = ops.prefill(qd, kd, vd, S, R, W)
    sout, slse = ops.streaming(qd, kd, vd, S, R)
    torch.cuda.synchronize()
    to, tl, tr = _tol(dtype)
    assert_close("out", np64(out), ref["out"], to)
    assert_close("lse", np64(lse), ref["lse"], tl)
    assert_close("lazy_rows", np64(rows), ref["lazy_rows"], tr)
    assert_close("lazy_ratio", np64(ratio), ref["lazy_ratio"], tr)
    assert_close("sout", np64(sout), ref["sout"], to)
    assert_close("slse", np64(slse), ref["slse"], tl)
    # the spikes do move the maxima: some LSE lie far above ln(i + 1) + a few
    assert float(np.max(ref["lse"])) > 20.0


@pytest.mark.parametrize("D", [128, 64])
def test_large_grid_with_score_spikes(D):
    """The 8-wave, 128-key shape (a grid of at least four of its workgroups
    per CU) and streaming on the same tensors, on sampled rows of every head
    around and after each spike."""
    B, N, Hq, Hkv, S, R, W = 1, 6140, 64, 8, 4, 300, 48
    spikes = _spikes(N, (1000, 1023, 1024, 2047, 4097, 5500, 6100))
    print(f"spiky large-grid prefill D{D} N{N} Hq{Hq} Hkv{Hkv}, {len(spikes)} spikes", flush=True)
    q, k, v = synth.qkv(B, N, Hq, Hkv, D, 81 + D, torch.bfloat16, device=DEV, spikes=spikes)
    out, lse, rows, ratio = ops.prefill(q, k, v, S, R, W)
    sout, slse = ops.streaming(q, k, v, S, R)
    torch.cuda.synchronize()
    G = Hq // Hkv
    near = np.concatenate([np.arange(p, p + 40) for p, _ in spikes] + [np.arange(N - W, N)])
    rng = np.random.default_rng(D)
    for h in range(Hq):
        pos = np.unique(np.concatenate([near[near < N], rng.integers(0, N, 8)])).astype(np.int32)
        pt = torch.as_tensor(pos, device=DEV, dtype=torch.long)
        r = oracle.rows(np64(k[0, h // G]), np64(v[0, h // G]), pos, np64(q[0, h][pt]), S=S, R=R)
        assert_close(f"out h{h}", np64(out[0, h][pt]), r["out"], TOL_BF16_OUT)
        assert_close(f"lse h{h}", np64(lse[0, h][pt]), r["lse"], TOL_BF16_LSE)
        assert_close(f"stream out h{h}", np64(sout[0, h][pt]), r["sout"], TOL_BF16_OUT)
        assert_close(f"stream lse h{h}", np64(slse[0, h][pt]), r["slse"], TOL_BF16_LSE)
        obs = pos >= N - W
        assert_close(f"lazy rows h{h}", np64(rows[0, h]), r["lazy"][obs], TOL_BF16_RATIO)
        assert abs(float(ratio[0, h]) - r["lazy"][obs].mean()) <= TOL_BF16_RATIO


def test_varlen_prefill_with_score_spikes():
    N, Hq, Hkv, D, S, R, W, lens = 500, 8, 2, 128, 4, 90, 24, [500, 301, 130, 64]
    print(f"spiky varlen prefill N{N} lens {lens}", flush=True)
    B = len(lens)
    q, k, v = synth.qkv(B, N, Hq, Hkv, D, 91, torch.bfloat16, spikes=_spikes(N))
    ref = oracle.prefill_varlen(np64(q), np64(k), np64(v), lens, S=S, R=R, W=W, streaming=True)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lens_d = torch.tensor(lens, device=DEV, dtype=torch.int32)
    out = torch.empty_like(qd)
    lse = torch.empty((B, Hq, N), device=DEV, dtype=torch.float32)
    rows = torch.empty((B, Hq, W), device=DEV, dtype=torch.float32)
    ratio = torch.empty((B, Hq), device=DEV, dtype=torch.float32)
    api.lt_prefill_attn_lse_lazy_varlen(qd, kd, vd, out, lse, lens_d, S, R, W, rows, ratio)
    sout = torch.empty_like(qd)
    slse = torch.empty((B, Hq, N), device=DEV, dtype=torch.float32)
    api.lt_streaming_attn_varlen(qd, kd, vd, sout, slse, lens_d, S, R)
    torch.cuda.synchronize()
    got_rows = np64(rows)
    for b, n in enumerate(lens):
        assert_close(f"out b{b}", np64(out[b, :, :n]), ref["out"][b, :, :n], TOL_BF16_OUT)
        assert_close(f"lse b{b}", np64(lse[b, :, :n]), ref["lse"][b, :, :n], TOL_BF16_LSE)
        assert_close(f"stream out b{b}", np64(sout[b, :, :n]), ref["sout"][b, :, :n], TOL_BF16_OUT)
        assert_close(f"stream lse b{b}", np64(slse[b, :, :n]), ref["slse"][b, :, :n], TOL_BF16_LSE)
        w = min(W, n)   # a short sequence's observed rows sit at the end of its W slots
        assert_close(f"lazy rows b{b}", got_rows[b, :, W - w:], ref["lazy_rows"][b, :, W - w:], TOL_BF16_RATIO)
        assert_close(f"lazy ratio b{b}", np64(ratio[b]), ref["lazy_ratio"][b], TOL_BF16_RATIO)


@pytest.mark.parametrize("L,dtype", [(5000, torch.bfloat16), (100000, torch.bfloat16), (3000, torch.float32)])
def test_decode_with_score_spikes(L, dtype):
    """Split-KV decode: spikes in different splits of the cache, one in the
    last key; the LSE merge must weigh the splits by their own maxima."""
    B, Hq, Hkv, D = 2, 10, 2, 128
    spikes = [(p, 16.0 if i % 2 == 0 else 100.0) for i, p in enumerate(sorted({0, 63, 64, L // 3, L // 2 + 1, L - 1}))]
    print(f"spiky decode B{B} Hq{Hq} Hkv{Hkv} D{D} L{L} {dtype}", flush=True)
    g = torch.Generator().manual_seed(95)
    q = torch.randn(B, Hq, D, generator=g)
    k = torch.randn(B, Hkv, L, D, generator=g)
    v = torch.randn(B, Hkv, L, D, generator=g)
    for p, f in spikes:
        k[:, :, p, :] *= f
    q, k, v = q.to(dtype), k.to(dtype), v.to(dtype)
    ref = oracle.decode(np64(q), np64(k), np64(v))
    out, lse = ops.decode(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    to, tl, _ = _tol(dtype)
    assert_close("out", np64(out), ref["out"], to)
    assert_close("lse", np64(lse), ref["lse"], tl)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_extreme_spikes_within_the_fp32_dot_product_bound(dtype):
    """Keys scaled by 10^4 (a spike of 100 applied twice) put logits in the
    thousands.  There the absolute LSE tolerances (1e-3, 1e-4) lie below what
    fp32 resolves: a plain fp32 reference misses them by as much.  The bound
    the arithmetic fixes is the forward error of an fp32 dot product,
    |fl(q.k) - q.k| <= gamma_D sum_d |q_d k_d| with gamma_D = D u / (1 - D u),
    u = 2^-24; the LSE is 1-Lipschitz in the max norm of a row's scores, so
    LSE_i may err by gamma_D max_{j<=i} sum_d |q_id k_jd| / sqrt(D) plus a few
    units of its own last place, on top of the usual tolerance.  Scores off by
    at most Delta move each weight exp(s - LSE) by a factor within
    exp(+-2 Delta), so an output row may err by 2 Delta max|v| on top of its
    tolerance (for bf16 inputs 3e-2: the bf16 tolerance plus the rounding of
    bf16 weights).  The ratio keeps the usual tolerance."""
    B, N, Hq, Hkv, D, S, R, W = 1, 800, 12, 3, 64, 4, 200, 100
    spikes = [(37, 100.0), (37, 100.0), (300, 100.0), (301, 100.0), (650, 100.0), (650, 100.0), (790, 16.0)]
    print(f"extreme spikes {dtype}", flush=True)
    q, k, v = synth.qkv(B, N, Hq, Hkv, D, 201, dtype, spikes=spikes)
    ref = oracle.prefill(np64(q), np64(k), np64(v), S=S, R=R, W=W, streaming=True)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse, rows, ratio = ops.prefill(qd, kd, vd, S, R, W)
    sout, slse = ops.streaming(qd, kd, vd, S, R)
    torch.cuda.synchronize()
    assert float(np.abs(ref["lse"]).max()) > 1e3
    u = 2.0 ** -24
    gamma = D * u / (1 - D * u)
    G = Hq // Hkv
    qa, ka = np.abs(np64(q)), np.abs(np64(k))
    tl = TOL_F32 if dtype == torch.float32 else TOL_BF16_LSE
    to = TOL_F32 if dtype == torch.float32 else 3e-2
    vmax = float(np.abs(np64(v)).max())
    for h in range(Hq):
        mag = qa[0, h] @ ka[0, h // G].T / np.sqrt(D)            # sum_d |q_id k_jd| / sqrt(D)
        delta = gamma * np.where(np.tri(N, dtype=bool), mag, 0.0).max(axis=1)
        for name, got, want in (("lse", lse, ref["lse"]), ("slse", slse, ref["slse"])):
            g_ = np64(got)[0, h]
            assert np.all(np.isfinite(g_))
            bound = tl + delta + 8 * u * np.abs(want[0, h])
            err = np.abs(g_ - want[0, h])
            assert np.all(err <= bound), f"{name} h{h}: max err/bound {(err / bound).max():.2f}"
        for name, got, want in (("out", out, ref["out"]), ("sout", sout, ref["sout"])):
            err = np.abs(np64(got)[0, h] - want[0, h]).max(axis=1)
            bound = to + 2 * delta * vmax
            assert np.all(err <= bound), f"{name} h{h}: max err/bound {(err / bound).max():.2f}"
    tr = TOL_F32 if dtype == torch.float32 else TOL_BF16_RATIO
    assert_close("lazy_ratio", np64(ratio), ref["lazy_ratio"], tr)
