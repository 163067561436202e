"""GPU parity at lengths beyond the workloads': a prefill of about 128K tokens
with a ragged tail (row and key indices past 2^16 and 2^17, the 8-wave
full-attention shape) and decode over contexts of about a million keys, both
against the fp64 oracle (sampled rows for the prefill, every output for the
decode)."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_causal_amd import ops, synth
from helpers import TOL_BF16_LSE, TOL_BF16_OUT, TOL_BF16_RATIO, assert_close, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_prefill_128k_tokens_sampled_rows():
    B, N, Hq, Hkv, D, S, R, W = 1, (1 << 17) - 37, 8, 1, 128, 4, 1020, 128
    print(f"prefill B{B} N{N} Hq{Hq} Hkv{Hkv} D{D} S{S} R{R} W{W}", flush=True)
    q, k, v = synth.qkv(B, N, Hq, Hkv, D, seed=71, device=DEV, sink_tokens=4, sink_scale=3.0)
    out, lse, rows, ratio = ops.prefill(q, k, v, S, R, W)
    sout, slse = ops.streaming(q, k, v, S, R)
    torch.cuda.synchronize()
    kh, vh = np64(k[0, 0]), np64(v[0, 0])
    rng = np.random.default_rng(71)
    # Positions around 2^16 and around the last tile boundary before N - W.
    edges = {(1 << 16) - 1, 1 << 16, (1 << 16) + 1, 98303, 98304, N - W - 1, N - 1025, N - 1024}
    for h in range(Hq):
        pos = set(range(N - W, N)) | set(range(16)) | edges | set(int(x) for x in rng.integers(0, N, 16))
        pos = np.array(sorted(pos), dtype=np.int32)
        pt = torch.as_tensor(pos, device=DEV, dtype=torch.long)
        r = oracle.rows(kh, vh, pos, np64(q[0, h][pt]), S=S, R=R)
        assert_close(f"out h{h}", np64(out[0, h][pt]), r["out"], TOL_BF16_OUT)
        assert_close(f"lse h{h}", np64(lse[0, h][pt]), r["lse"], TOL_BF16_LSE)
        assert_close(f"stream out h{h}", np64(sout[0, h][pt]), r["sout"], TOL_BF16_OUT)
        assert_close(f"stream lse h{h}", np64(slse[0, h][pt]), r["slse"], TOL_BF16_LSE)
        obs = pos >= N - W
        assert_close(f"lazy rows h{h}", np64(rows[0, h]), r["lazy"][obs], TOL_BF16_RATIO)
        assert abs(float(ratio[0, h]) - r["lazy"][obs].sum() / W) <= TOL_BF16_RATIO


def test_decode_over_a_million_keys():
    B, Hq, Hkv, D, L = 2, 8, 1, 128, (1 << 20) + 7
    lens = [L, 333331]
    print(f"decode B{B} Hq{Hq} Hkv{Hkv} D{D} L{L} lens {lens}", flush=True)
    q = synth.normal((B, Hq, D), 73, torch.bfloat16, device=DEV)
    k = synth.normal((B, Hkv, L, D), 74, torch.bfloat16, device=DEV)
    v = synth.normal((B, Hkv, L, D), 75, torch.bfloat16, device=DEV)
    out, lse = ops.decode(q, k, v)
    vout, vlse = ops.decode_varlen(q, k, v, lens)
    torch.cuda.synchronize()
    qh, kh, vh = np64(q), np64(k), np64(v)
    ref = oracle.decode(qh, kh, vh)
    assert_close("out", np64(out), ref["out"], TOL_BF16_OUT)
    assert_close("lse", np64(lse), ref["lse"], TOL_BF16_LSE)
    vref = oracle.decode_varlen(qh, kh, vh, lens)
    assert_close("varlen out", np64(vout), vref["out"], TOL_BF16_OUT)
    assert_close("varlen lse", np64(vlse), vref["lse"], TOL_BF16_LSE)
