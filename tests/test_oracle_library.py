"""Pin the oracle against independent library routines (torch fp64 on CPU).

* attention output: torch scaled_dot_product_attention (causal, and with an
  explicit boolean mask for the sink + recent set), K/V heads repeated to
  the GQA map h -> h // (Hq/Hkv);
* LSE: torch.logsumexp over the masked score matrix from torch.matmul.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _sdpa(q, k, v, mask=None, causal=False):
    G = q.shape[1] // k.shape[1]
    kk = k.repeat_interleave(G, dim=1)
    vv = v.repeat_interleave(G, dim=1)
    return F.scaled_dot_product_attention(q, kk, vv, attn_mask=mask, is_causal=causal)


def _scores(q, k):
    G = q.shape[1] // k.shape[1]
    kk = k.repeat_interleave(G, dim=1)
    return torch.matmul(q, kk.transpose(-1, -2)) / math.sqrt(q.shape[-1])


def _stream_mask(N, S, R):
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    return (j <= i) & ((j < S) | (j > i - R))


@pytest.mark.parametrize("B,N,Hq,Hkv,D,S,R,seed", [(1, 64, 6, 2, 16, 4, 10, 0),
                                                   (2, 97, 8, 8, 8, 0, 20, 1),
                                                   (1, 50, 5, 1, 32, 3, 1, 2)])
def test_against_torch(B, N, Hq, Hkv, D, S, R, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, N, D, generator=g, dtype=torch.float64)
    k = torch.randn(B, Hkv, N, D, generator=g, dtype=torch.float64)
    v = torch.randn(B, Hkv, N, D, generator=g, dtype=torch.float64)
    got = oracle.prefill(q.numpy(), k.numpy(), v.numpy(), S=S, R=R, W=N, streaming=True)
    np.testing.assert_allclose(got["out"], _sdpa(q, k, v, causal=True).numpy(), atol=1e-12)
    sc = _scores(q, k)
    causal = torch.ones(N, N, dtype=torch.bool).tril()
    lse = torch.logsumexp(sc.masked_fill(~causal, -math.inf), dim=-1)
    np.testing.assert_allclose(got["lse"], lse.numpy(), atol=1e-12)
    m = _stream_mask(N, S, R)
    np.testing.assert_allclose(got["sout"], _sdpa(q, k, v, mask=m).numpy(), atol=1e-12)
    slse = torch.logsumexp(sc.masked_fill(~m, -math.inf), dim=-1)
    np.testing.assert_allclose(got["slse"], slse.numpy(), atol=1e-12)
    # per-row lazy ratio: masked softmax mass, from torch.softmax
    P = torch.softmax(sc.masked_fill(~causal, -math.inf), dim=-1)
    r = (P * m).sum(-1)
    np.testing.assert_allclose(got["lazy_rows"], r.numpy(), atol=1e-12)


def test_decode_against_torch():
    g = torch.Generator().manual_seed(5)
    q = torch.randn(3, 10, 1, 16, generator=g, dtype=torch.float64)
    k = torch.randn(3, 2, 77, 16, generator=g, dtype=torch.float64)
    v = torch.randn(3, 2, 77, 16, generator=g, dtype=torch.float64)
    got = oracle.decode(q[:, :, 0].numpy(), k.numpy(), v.numpy())
    np.testing.assert_allclose(got["out"], _sdpa(q, k, v)[:, :, 0].numpy(), atol=1e-12)
    lse = torch.logsumexp(_scores(q, k)[:, :, 0], dim=-1)
    np.testing.assert_allclose(got["lse"], lse.numpy(), atol=1e-12)
