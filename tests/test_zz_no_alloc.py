"""lt_hybrid_decode_attn_noalloc (the decode call that allocates nothing)
against lt_hybrid_decode_attn, through the C ABI: two calls in a row, the
second smaller, each bit-identical to the call with a caller's workspace
(same kernels, same split of the keys) and within the bf16 tolerance of the
oracle; then a size whose partial states exceed the library's scratch array
is refused before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_causal_amd import _lib, ops
from helpers import TOL_BF16_LSE, TOL_BF16_OUT, assert_close, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _view(t):
    return _lib.LtView(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _noalloc(q, k, v, kv_len, out, lse):
    B, Hq, D = q.shape
    st = torch.cuda.current_stream().cuda_stream
    return _lib.lib().lt_hybrid_decode_attn_noalloc(B, Hq, k.shape[1], D, _lib.LT_BF16, 0.0, q.data_ptr(),
                                                    _view(k), _view(v), kv_len, out.data_ptr(),
                                                    lse.data_ptr(), st)


def test_noalloc_decode_matches_workspace_call():
    torch.manual_seed(0)
    cases = [(8, 40, 8, 128, 100000, 100000),   # a full decode100k-shaped layer
             (3, 20, 4, 64, 1500, 1500),        # smaller: fewer splits, other head dim
             (2, 16, 2, 128, 700, 650)]         # cache longer than the attended rows
    for B, Hq, Hkv, D, rows, kv_len in cases:
        print(f"noalloc decode B{B} Hq{Hq} Hkv{Hkv} D{D} kv_len {kv_len}", flush=True)
        g = torch.Generator(device=DEV).manual_seed(B * 1000 + kv_len)
        q = torch.randn(B, Hq, D, generator=g, device=DEV).to(torch.bfloat16)
        k = torch.randn(B, Hkv, rows, D, generator=g, device=DEV).to(torch.bfloat16)
        v = torch.randn(B, Hkv, rows, D, generator=g, device=DEV).to(torch.bfloat16)
        out = torch.full((B, Hq, D), 7.0, device=DEV, dtype=torch.bfloat16)
        lse = torch.full((B, Hq), 7.0, device=DEV, dtype=torch.float32)
        assert _noalloc(q, k, v, kv_len, out, lse) == _lib.LT_OK, _lib.lib().lt_last_error()
        want_out, want_lse = ops.decode(q, k, v, kv_len)
        torch.cuda.synchronize()
        assert torch.equal(out, want_out) and torch.equal(lse, want_lse)
        G = Hq // Hkv
        for b, hk in [(0, 0), (B - 1, Hkv - 1)]:
            r = oracle.decode(np64(q[b:b + 1, hk * G:(hk + 1) * G]), np64(k[b:b + 1, hk:hk + 1, :kv_len]),
                              np64(v[b:b + 1, hk:hk + 1, :kv_len]))
            assert_close(f"out b{b} hk{hk}", np64(out[b:b + 1, hk * G:(hk + 1) * G]), r["out"], TOL_BF16_OUT)
            assert_close(f"lse b{b} hk{hk}", np64(lse[b:b + 1, hk * G:(hk + 1) * G]), r["lse"], TOL_BF16_LSE)


def test_noalloc_decode_refuses_sizes_beyond_its_scratch():
    """1024 sequences of 64 keys, 16 query heads per KV head: one split per
    sequence, 2047 partial-state slots of [16, 130] fp32, about 17 MB, more
    than the scratch array; refused before any launch, outputs untouched."""
    B, Hq, Hkv, D, kv_len = 1024, 16, 1, 128, 64
    n = ctypes.c_size_t()
    assert _lib.lib().lt_hybrid_decode_workspace_bytes(B, Hq, Hkv, D, kv_len, ctypes.byref(n)) == 0
    assert n.value > _lib.LT_DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, Hq, D, device=DEV, dtype=torch.bfloat16)
    k = torch.zeros(B, Hkv, kv_len, D, device=DEV, dtype=torch.bfloat16)
    out = torch.full_like(q, 3.0)
    lse = torch.full((B, Hq), 3.0, device=DEV)
    rc = _noalloc(q, k, k, kv_len, out, lse)
    torch.cuda.synchronize()
    assert rc == _lib.LT_ERR_WORKSPACE
    assert bool((out == 3.0).all()) and bool((lse == 3.0).all())
