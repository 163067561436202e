"""Allocating conveniences over the C-ABI binding (outputs are new tensors on
the inputs' device; every computation happens in liblt.so)."""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import api


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, S: int, R: int, W: int,
            scale: float = 0.0, stream=None):
    """Returns (out, lse, lazy_rows, lazy_ratio); the last two are None if W == 0."""
    B, Hq, N, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, N, device=q.device, dtype=torch.float32)
    rows = ratio = None
    if W > 0:
        rows = torch.empty(B, Hq, W, device=q.device, dtype=torch.float32)
        ratio = torch.empty(B, Hq, device=q.device, dtype=torch.float32)
    api.lt_prefill_attn_lse_lazy(q, k, v, out, lse, S, R, W, rows, ratio, scale, stream)
    return out, lse, rows, ratio


def streaming(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, S: int, R: int,
              with_lse: bool = True, scale: float = 0.0, stream=None):
    B, Hq, N, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, N, device=q.device, dtype=torch.float32) if with_lse else None
    api.lt_streaming_attn(q, k, v, out, lse, S, R, scale, stream)
    return out, lse


def decode_workspace(B: int, Hq: int, Hkv: int, D: int, kv_len: int, device) -> torch.Tensor:
    n = api.lt_hybrid_decode_workspace_bytes(B, Hq, Hkv, D, kv_len)
    return torch.empty(max(n, 16), device=device, dtype=torch.uint8)


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           kv_len: Optional[int] = None, ws: Optional[torch.Tensor] = None, scale: float = 0.0,
           stream=None):
    B, Hq, D = q.shape
    L = k_cache.shape[2] if kv_len is None else kv_len
    if ws is None:
        ws = decode_workspace(B, Hq, k_cache.shape[1], D, L, q.device)
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, device=q.device, dtype=torch.float32)
    api.lt_hybrid_decode_attn(q, k_cache, v_cache, L, out, lse, ws, scale, stream)
    return out, lse


def compact(k_full: torch.Tensor, v_full: torch.Tensor, S: int, R: int, stream=None,
            slots: Optional[int] = None):
    """Streaming cache of min(N, S+R) rows (or `slots` >= that many, e.g. S+R
    for a cache that decode will keep appending to)."""
    B, Hkv, N, D = k_full.shape
    rows = min(N, S + R) if slots is None else max(slots, min(N, S + R))
    ks = torch.empty(B, Hkv, rows, D, device=k_full.device, dtype=k_full.dtype)
    vs = torch.empty_like(ks)
    api.lt_compact_kv_streaming(k_full, v_full, ks, vs, S, R, stream)
    return ks, vs


def stream_append(k_stream: torch.Tensor, v_stream: torch.Tensor, k_new: torch.Tensor,
                  v_new: torch.Tensor, S: int, R: int, pos: int, stream=None) -> int:
    """Append the token at position pos; returns the kv_len to decode with."""
    api.lt_stream_cache_append(k_stream, v_stream, k_new.contiguous(), v_new.contiguous(), S, R, pos,
                               stream)
    return min(pos + 1, S + R)


def _device_lens(lens, device) -> torch.Tensor:
    if isinstance(lens, torch.Tensor):
        return lens.to(device=device, dtype=torch.int32).contiguous()
    return torch.tensor(list(lens), device=device, dtype=torch.int32)


def prefill_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens, S: int, R: int, W: int,
                   scale: float = 0.0, stream=None):
    """Padded variable-length batch; seq_lens: [B] lengths (list or tensor).
    Returns (out, lse, lazy_rows, lazy_ratio); rows past a sequence's length
    are left as torch.empty made them."""
    B, Hq, N, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, N, device=q.device, dtype=torch.float32)
    rows = ratio = None
    if W > 0:
        rows = torch.empty(B, Hq, W, device=q.device, dtype=torch.float32)
        ratio = torch.empty(B, Hq, device=q.device, dtype=torch.float32)
    api.lt_prefill_attn_lse_lazy_varlen(q, k, v, out, lse, _device_lens(seq_lens, q.device), S, R, W, rows,
                                        ratio, scale, stream)
    return out, lse, rows, ratio


def decode_varlen(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_lens,
                  max_kv_len: Optional[int] = None, ws: Optional[torch.Tensor] = None, scale: float = 0.0,
                  stream=None):
    """Decode with per-sequence context lengths kv_lens [B] (<= max_kv_len,
    by default the cache rows)."""
    B, Hq, D = q.shape
    L = k_cache.shape[2] if max_kv_len is None else max_kv_len
    if ws is None:
        ws = decode_workspace(B, Hq, k_cache.shape[1], D, L, q.device)
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, device=q.device, dtype=torch.float32)
    api.lt_hybrid_decode_attn_varlen(q, k_cache, v_cache, _device_lens(kv_lens, q.device), L, out, lse, ws,
                                     scale, stream)
    return out, lse



def decode_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, block_table, kv_lens,
                 ws: Optional[torch.Tensor] = None, scale: float = 0.0, stream=None):
    """Decode over paged caches: pools [num_pages, Hkv, page_size, D], a
    block table [B, max_pages] (tensor or nested lists) and lengths [B]."""
    B, Hq, D = q.shape
    table = block_table if isinstance(block_table, torch.Tensor) else torch.tensor(block_table, dtype=torch.int32)
    table = table.to(device=q.device, dtype=torch.int32).contiguous()
    if ws is None:
        ws = decode_workspace(B, Hq, k_pool.shape[1], D, table.shape[1] * k_pool.shape[2], q.device)
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, device=q.device, dtype=torch.float32)
    api.lt_hybrid_decode_attn_paged(q, k_pool, v_pool, table, _device_lens(kv_lens, q.device), out, lse, ws,
                                    scale, stream)
    return out, lse

def prefill_emit(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, S: int, R: int, W: int, seq_lens=None,
                 slots: Optional[int] = None, scale: float = 0.0, stream=None):
    """Prefill + LSE + lazy ratio that also writes the streaming slice.
    Returns (out, lse, lazy_rows, lazy_ratio, k_stream, v_stream); the
    streaming cache has min(N, S+R) rows, or `slots` (>= that) for a cache
    that decode will keep appending to."""
    B, Hq, N, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, N, device=q.device, dtype=torch.float32)
    rows = ratio = None
    if W > 0:
        rows = torch.empty(B, Hq, W, device=q.device, dtype=torch.float32)
        ratio = torch.empty(B, Hq, device=q.device, dtype=torch.float32)
    n_slots = min(N, S + R) if slots is None else max(slots, min(N, S + R))
    ks = torch.empty(B, k.shape[1], n_slots, D, device=q.device, dtype=q.dtype)
    vs = torch.empty_like(ks)
    lens = None if seq_lens is None else _device_lens(seq_lens, q.device)
    api.lt_prefill_attn_lse_lazy_emit(q, k, v, out, lse, S, R, W, rows, ratio, ks, vs, lens, scale, stream)
    return out, lse, rows, ratio, ks, vs
