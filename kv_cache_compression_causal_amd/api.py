"""Thin Python binding of include/lt.h, one function per C entry point.

Marshalling only: tensors become (device pointer, element strides), the
stream is torch's current HIP stream unless one is given, and a non-zero
status raises LtError.  Every step of the computation runs in liblt.so.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

from ._lib import LT_BF16, LT_F32, LtShape, LtView, check, lib

_DTYPES = {torch.bfloat16: LT_BF16, torch.float32: LT_F32}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def _dev(t: torch.Tensor) -> int:
    """Device address of a tensor on the current GPU (the kernels run there:
    a host or other-device pointer would fault instead of failing)."""
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"tensor on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    return t.data_ptr()


def _view(t: torch.Tensor) -> LtView:
    """[B, H, rows, D] tensor -> lt_view (head dim must be contiguous)."""
    if t.dim() != 4:
        raise ValueError("expected a [B, H, rows, D] tensor")
    if t.stride(3) != 1:
        raise ValueError("head dim must be contiguous")
    return LtView(_dev(t), t.stride(0), t.stride(1), t.stride(2))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else _dev(t)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _shape(q: torch.Tensor, k: torch.Tensor, scale: float) -> LtShape:
    B, Hq, N, D = q.shape
    return LtShape(B, N, Hq, k.shape[1], D, _dtype_code(q), float(scale))


def _same_dtype(*ts: torch.Tensor) -> None:
    if len({t.dtype for t in ts}) != 1:
        raise TypeError("q, k, v and out must share one dtype")


def _lazy_outputs(rows: Optional[torch.Tensor], ratio: Optional[torch.Tensor], B: int, Hq: int, W: int):
    """With W > 0 the kernels write rows [B, Hq, W] and ratio [B, Hq] (fp32,
    contiguous); W == 0 writes neither, and both are passed as NULL."""
    if W <= 0:
        return None, None
    for t, shape, name in ((rows, (B, Hq, W), "lazy_rows"), (ratio, (B, Hq), "lazy_ratio")):
        if t is None:
            continue  # the library reports the missing buffer
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != shape:
            raise ValueError(f"{name} must be a contiguous float32 {list(shape)} tensor")
    return _ptr(rows), _ptr(ratio)


def lt_prefill_attn_lse_lazy(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                             lse: torch.Tensor, S: int, R: int, W: int,
                             lazy_rows: Optional[torch.Tensor] = None,
                             lazy_ratio: Optional[torch.Tensor] = None, scale: float = 0.0,
                             stream=None) -> None:
    _same_dtype(q, k, v, out)
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2] or out.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v, out")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must be a contiguous float32 [B, Hq, N] tensor")
    shp = _shape(q, k, scale)
    rows, ratio = _lazy_outputs(lazy_rows, lazy_ratio, q.shape[0], q.shape[1], W)
    check(lib().lt_prefill_attn_lse_lazy(ctypes.byref(shp), _view(q), _view(k), _view(v), _view(out),
                                         _ptr(lse), S, R, W, rows, ratio, _stream(stream)))


def lt_streaming_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                      lse: Optional[torch.Tensor], S: int, R: int, scale: float = 0.0,
                      stream=None) -> None:
    _same_dtype(q, k, v, out)
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2] or out.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v, out")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != tuple(q.shape[:3])):
        raise ValueError("lse must be a contiguous float32 [B, Hq, N] tensor")
    shp = _shape(q, k, scale)
    check(lib().lt_streaming_attn(ctypes.byref(shp), _view(q), _view(k), _view(v), _view(out),
                                  _ptr(lse), S, R, _stream(stream)))


def lt_hybrid_decode_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, kv_len: int) -> int:
    n = ctypes.c_size_t()
    check(lib().lt_hybrid_decode_workspace_bytes(B, Hq, Hkv, D, kv_len, ctypes.byref(n)))
    return n.value


def lt_hybrid_decode_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          kv_len: int, out: torch.Tensor, lse: Optional[torch.Tensor],
                          ws: torch.Tensor, scale: float = 0.0, stream=None) -> None:
    """q, out [B, Hq, D] contiguous; caches [B, Hkv, >=kv_len, D]; ws from
    lt_hybrid_decode_workspace_bytes (any dtype, contiguous)."""
    if not (q.is_contiguous() and out.is_contiguous() and ws.is_contiguous()):
        raise ValueError("q, out and ws must be contiguous")
    _same_dtype(q, k_cache, v_cache, out)
    B, Hq, D = q.shape
    if tuple(out.shape) != (B, Hq, D) or k_cache.shape[0] != B or k_cache.shape[3] != D \
            or k_cache.shape[2] < kv_len or v_cache.shape[:2] != k_cache.shape[:2] \
            or v_cache.shape[2] < kv_len or v_cache.shape[3] != D:
        raise ValueError("decode shape mismatch")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, Hq)):
        raise ValueError("lse must be a contiguous float32 [B, Hq] tensor")
    check(lib().lt_hybrid_decode_attn(B, Hq, k_cache.shape[1], D, _dtype_code(q), float(scale),
                                      _ptr(q), _view(k_cache), _view(v_cache), int(kv_len),
                                      _ptr(out), _ptr(lse), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)))


def lt_compact_kv_streaming(k_full: torch.Tensor, v_full: torch.Tensor, k_stream: torch.Tensor,
                            v_stream: torch.Tensor, S: int, R: int, stream=None) -> None:
    B, Hkv, N, D = k_full.shape
    rows = min(N, S + R)
    for t in (v_full,):
        if t.shape != k_full.shape:
            raise ValueError("k_full / v_full shape mismatch")
    for t in (k_stream, v_stream):
        if t.shape[0] != B or t.shape[1] != Hkv or t.shape[2] < rows or t.shape[3] != D:
            raise ValueError("streaming cache too small")
    _same_dtype(k_full, v_full, k_stream, v_stream)
    check(lib().lt_compact_kv_streaming(_view(k_full), _view(v_full), _view(k_stream),
                                        _view(v_stream), B, Hkv, N, D, _dtype_code(k_full), S, R,
                                        _stream(stream)))


def lt_stream_cache_append(k_stream: torch.Tensor, v_stream: torch.Tensor, k_new: torch.Tensor,
                           v_new: torch.Tensor, S: int, R: int, pos: int, stream=None) -> None:
    """k_new, v_new [B, Hkv, D] contiguous: the token at position pos; written
    into its slot of the streaming cache [B, Hkv, >=min(pos+1, S+R), D]."""
    B, Hkv, rows, D = k_stream.shape
    if not (k_new.is_contiguous() and v_new.is_contiguous()):
        raise ValueError("k_new and v_new must be contiguous")
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D) \
            or v_stream.shape != k_stream.shape:
        raise ValueError("append shape mismatch")
    if rows < min(pos + 1, S + R):
        raise ValueError("streaming cache has too few rows for this position")
    _same_dtype(k_stream, v_stream, k_new, v_new)
    check(lib().lt_stream_cache_append(_view(k_stream), _view(v_stream), _ptr(k_new),
                                       _ptr(v_new), B, Hkv, D, _dtype_code(k_stream), S, R,
                                       int(pos), _stream(stream)))


def _lens(t: torch.Tensor, B: int, name: str) -> int:
    """Per-sequence length / position array: a contiguous int32 [B] device tensor."""
    if t.dtype != torch.int32 or t.dim() != 1 or t.numel() != B or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous int32 [B] device tensor")
    return _dev(t)


def lt_prefill_attn_lse_lazy_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                                    lse: torch.Tensor, seq_lens: torch.Tensor, S: int, R: int, W: int,
                                    lazy_rows: Optional[torch.Tensor] = None,
                                    lazy_ratio: Optional[torch.Tensor] = None, scale: float = 0.0,
                                    stream=None) -> None:
    """Padded variable-length batch: q [B,Hq,N,D] etc. padded to N; seq_lens
    [B] int32 on the device."""
    _same_dtype(q, k, v, out)
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2] or out.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v, out")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must be a contiguous float32 [B, Hq, N] tensor")
    shp = _shape(q, k, scale)
    rows, ratio = _lazy_outputs(lazy_rows, lazy_ratio, q.shape[0], q.shape[1], W)
    check(lib().lt_prefill_attn_lse_lazy_varlen(ctypes.byref(shp), _lens(seq_lens, q.shape[0], "seq_lens"),
                                                _view(q), _view(k), _view(v), _view(out), _ptr(lse), S, R,
                                                W, rows, ratio, _stream(stream)))


def lt_prefill_attn_lse_lazy_emit(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                                  lse: torch.Tensor, S: int, R: int, W: int, lazy_rows: Optional[torch.Tensor],
                                  lazy_ratio: Optional[torch.Tensor], k_stream: torch.Tensor,
                                  v_stream: torch.Tensor, seq_lens: Optional[torch.Tensor] = None,
                                  scale: float = 0.0, stream=None) -> None:
    """Prefill + LSE + lazy ratio that also writes the layer's streaming
    slice into k_stream / v_stream [B, Hkv, >= min(N, S+R), D] (seq_lens:
    optional int32 [B] device lengths of a padded batch)."""
    _same_dtype(q, k, v, out, k_stream, v_stream)
    B, Hq, N, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or out.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v, out")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be a contiguous float32 [B, Hq, N] tensor")
    for t in (k_stream, v_stream):
        if t.dim() != 4 or t.shape[0] != B or t.shape[1] != k.shape[1] or t.shape[2] < min(N, S + R) \
                or t.shape[3] != D:
            raise ValueError("streaming cache must be [B, Hkv, >= min(N, S+R), D]")
    lens = None if seq_lens is None else _lens(seq_lens, B, "seq_lens")
    shp = _shape(q, k, scale)
    rows, ratio = _lazy_outputs(lazy_rows, lazy_ratio, B, Hq, W)
    check(lib().lt_prefill_attn_lse_lazy_emit(ctypes.byref(shp), lens, _view(q), _view(k), _view(v),
                                              _view(out), _ptr(lse), S, R, W, rows, ratio,
                                              _view(k_stream), _view(v_stream), _stream(stream)))


def lt_streaming_attn_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                             lse: Optional[torch.Tensor], seq_lens: torch.Tensor, S: int, R: int,
                             scale: float = 0.0, stream=None) -> None:
    _same_dtype(q, k, v, out)
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2] or out.shape != q.shape:
        raise ValueError("shape mismatch between q, k, v, out")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != tuple(q.shape[:3])):
        raise ValueError("lse must be a contiguous float32 [B, Hq, N] tensor")
    shp = _shape(q, k, scale)
    check(lib().lt_streaming_attn_varlen(ctypes.byref(shp), _lens(seq_lens, q.shape[0], "seq_lens"), _view(q),
                                         _view(k), _view(v), _view(out), _ptr(lse), S, R, _stream(stream)))


def lt_hybrid_decode_attn_varlen(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 kv_lens: torch.Tensor, max_kv_len: int, out: torch.Tensor,
                                 lse: Optional[torch.Tensor], ws: torch.Tensor, scale: float = 0.0,
                                 stream=None) -> None:
    """kv_lens [B] int32 on the device, each <= max_kv_len; ws sized by
    lt_hybrid_decode_workspace_bytes(..., max_kv_len)."""
    if not (q.is_contiguous() and out.is_contiguous() and ws.is_contiguous()):
        raise ValueError("q, out and ws must be contiguous")
    _same_dtype(q, k_cache, v_cache, out)
    B, Hq, D = q.shape
    if tuple(out.shape) != (B, Hq, D) or k_cache.shape[0] != B or k_cache.shape[3] != D \
            or k_cache.shape[2] < max_kv_len or v_cache.shape[:2] != k_cache.shape[:2] \
            or v_cache.shape[2] < max_kv_len or v_cache.shape[3] != D:
        raise ValueError("decode shape mismatch")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, Hq)):
        raise ValueError("lse must be a contiguous float32 [B, Hq] tensor")
    check(lib().lt_hybrid_decode_attn_varlen(B, Hq, k_cache.shape[1], D, _dtype_code(q), float(scale),
                                             _ptr(q), _view(k_cache), _view(v_cache),
                                             _lens(kv_lens, B, "kv_lens"), int(max_kv_len), _ptr(out),
                                             _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                             _stream(stream)))



def lt_hybrid_decode_attn_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                block_table: torch.Tensor, kv_lens: torch.Tensor, out: torch.Tensor,
                                lse: Optional[torch.Tensor], ws: torch.Tensor, scale: float = 0.0,
                                stream=None) -> None:
    """Paged caches: k_pool / v_pool [num_pages, Hkv, page_size, D] (any
    strides with D contiguous), block_table [B, max_pages] and kv_lens [B]
    int32 on the device; ws sized by lt_hybrid_decode_workspace_bytes(...,
    max_pages * page_size)."""
    if not (q.is_contiguous() and out.is_contiguous() and ws.is_contiguous()):
        raise ValueError("q, out and ws must be contiguous")
    _same_dtype(q, k_pool, v_pool, out)
    B, Hq, D = q.shape
    if tuple(out.shape) != (B, Hq, D) or k_pool.dim() != 4 or k_pool.shape[3] != D \
            or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("paged decode shape mismatch")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B \
            or not block_table.is_contiguous() or not block_table.is_cuda:
        raise ValueError("block_table must be a contiguous int32 [B, max_pages] device tensor")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, Hq)):
        raise ValueError("lse must be a contiguous float32 [B, Hq] tensor")
    num_pages, Hkv, page_size = k_pool.shape[:3]
    check(lib().lt_hybrid_decode_attn_paged(B, Hq, Hkv, D, _dtype_code(q), float(scale), _ptr(q),
                                            _view(k_pool), _view(v_pool), page_size, num_pages,
                                            _dev(block_table), block_table.shape[1],
                                            _lens(kv_lens, B, "kv_lens"), _ptr(out), _ptr(lse), _ptr(ws),
                                            ws.numel() * ws.element_size(), _stream(stream)))

def lt_compact_kv_streaming_varlen(k_full: torch.Tensor, v_full: torch.Tensor, k_stream: torch.Tensor,
                                   v_stream: torch.Tensor, seq_lens: torch.Tensor, S: int, R: int,
                                   stream=None) -> None:
    B, Hkv, N, D = k_full.shape
    rows = min(N, S + R)
    if v_full.shape != k_full.shape:
        raise ValueError("k_full / v_full shape mismatch")
    for t in (k_stream, v_stream):
        if t.shape[0] != B or t.shape[1] != Hkv or t.shape[2] < rows or t.shape[3] != D:
            raise ValueError("streaming cache too small")
    _same_dtype(k_full, v_full, k_stream, v_stream)
    check(lib().lt_compact_kv_streaming_varlen(_view(k_full), _view(v_full), _view(k_stream),
                                               _view(v_stream), B, Hkv, N, D, _dtype_code(k_full), S, R,
                                               _lens(seq_lens, B, "seq_lens"), _stream(stream)))


def lt_stream_cache_append_varlen(k_stream: torch.Tensor, v_stream: torch.Tensor, k_new: torch.Tensor,
                                  v_new: torch.Tensor, S: int, R: int, pos: torch.Tensor,
                                  stream=None) -> None:
    """pos [B] int32 on the device (negative: skip that sequence); the caches
    hold S + R slots."""
    B, Hkv, rows, D = k_stream.shape
    if not (k_new.is_contiguous() and v_new.is_contiguous()):
        raise ValueError("k_new and v_new must be contiguous")
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D) \
            or v_stream.shape != k_stream.shape:
        raise ValueError("append shape mismatch")
    if rows < S + R:
        raise ValueError("the streaming cache needs S + R slots")
    _same_dtype(k_stream, v_stream, k_new, v_new)
    check(lib().lt_stream_cache_append_varlen(_view(k_stream), _view(v_stream), _ptr(k_new),
                                              _ptr(v_new), B, Hkv, D, _dtype_code(k_stream), S, R,
                                              _lens(pos, B, "pos"), _stream(stream)))


def lt_kv_bytes(B: int, Hkv: int, N: int, D: int, dtype: int, S: int, R: int) -> Tuple[int, int]:
    full, stream = ctypes.c_int64(), ctypes.c_int64()
    check(lib().lt_kv_bytes(B, Hkv, N, D, dtype, S, R, ctypes.byref(full), ctypes.byref(stream)))
    return full.value, stream.value


class LazyQueue:
    """lt_lazy_queue_create_policy / _push / _destroy.  policy: LT_EVICT_AFTER_PUSH
    (0, the default) or LT_EVICT_BEFORE_PUSH (1)."""

    def __init__(self, L: int, C: int, policy: int = 0):
        h = ctypes.c_void_p()
        check(lib().lt_lazy_queue_create_policy(L, C, int(policy), ctypes.byref(h)))
        self._h = h

    def push(self, layer: int, score: float) -> int:
        ev = ctypes.c_int()
        check(lib().lt_lazy_queue_push(self._h, layer, float(score), ctypes.byref(ev)))
        return ev.value

    def push_ratios(self, layer: int, head_ratio) -> Tuple[int, float]:
        """Push with the score computed in the library from the layer's
        per-(batch, head) ratios (host, fp32).  Returns (evicted, score)."""
        hr = np.ascontiguousarray(np.asarray(head_ratio, dtype=np.float32).reshape(-1))
        ev = ctypes.c_int()
        sc = ctypes.c_double()
        check(lib().lt_lazy_queue_push_ratios(self._h, layer,
                                              hr.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                              hr.size, ctypes.byref(sc), ctypes.byref(ev)))
        return ev.value, sc.value

    def set_kv_bytes(self, full_bytes: int, stream_bytes: int, emit: bool = False) -> None:
        """Per-layer KV sizes for the queue's byte accounting (before the first push)."""
        check(lib().lt_lazy_queue_set_kv_bytes(self._h, int(full_bytes), int(stream_bytes), int(bool(emit))))

    def kv_bytes(self) -> Tuple[int, int]:
        """(retained, transient) KV bytes of the last push's step."""
        r, t = ctypes.c_int64(), ctypes.c_int64()
        check(lib().lt_lazy_queue_kv_bytes(self._h, ctypes.byref(r), ctypes.byref(t)))
        return r.value, t.value

    def close(self) -> None:
        if self._h:
            lib().lt_lazy_queue_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def lt_select_lazy_layers(head_ratio, C: int, policy: int = 0):
    """head_ratio [L, n] (host, fp32).  Returns (layer_score [L] float64,
    evicted_at_step [L] int32, is_streaming [L] uint8).  policy as for
    LazyQueue (lt_select_lazy_layers_policy)."""
    hr = np.ascontiguousarray(np.asarray(head_ratio, dtype=np.float32))
    if hr.ndim != 2:
        raise ValueError("head_ratio must be [L, n]")
    L, n = hr.shape
    score = np.empty(L, dtype=np.float64)
    ev = np.empty(L, dtype=np.int32)
    st = np.empty(L, dtype=np.uint8)
    check(lib().lt_select_lazy_layers_policy(
        hr.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), L, n, C, int(policy),
        score.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        ev.ctypes.data_as(ctypes.POINTER(ctypes.c_int)),
        st.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))))
    return score, ev, st


def lt_kv_accounting(evicted_at_step, full_bytes: int, stream_bytes: int, policy: int = 0,
                     emit: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Per-step (retained [L], transient [L]) KV bytes of a run from its
    evicted_at_step [L] (lt_kv_accounting)."""
    ev = np.ascontiguousarray(np.asarray(evicted_at_step, dtype=np.int32).reshape(-1))
    L = ev.size
    ret = np.empty(L, dtype=np.int64)
    tra = np.empty(L, dtype=np.int64)
    check(lib().lt_kv_accounting(ev.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), L, int(policy),
                                 int(full_bytes), int(stream_bytes), int(bool(emit)),
                                 ret.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                 tra.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
    return ret, tra


def lt_select_offline(head_ratio, C: int):
    """head_ratio [P, L, n] (host, fp32): per-(batch, head) lazy ratios of
    every layer on every prompt.  Returns (layer_score [L] float64, the mean
    over prompts; is_streaming [L] uint8)."""
    hr = np.ascontiguousarray(np.asarray(head_ratio, dtype=np.float32))
    if hr.ndim != 3:
        raise ValueError("head_ratio must be [P, L, n]")
    P, L, n = hr.shape
    score = np.empty(L, dtype=np.float64)
    st = np.empty(L, dtype=np.uint8)
    check(lib().lt_select_offline(hr.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), P, L, n, C,
                                  score.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                  st.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))))
    return score, st


def lt_probe_mfma_bf16(blocks: int, iters: int, sink: torch.Tensor, stream=None) -> float:
    """Launch the matrix-core probe; returns the FLOP it performs (the caller
    times it).  sink: float32 device tensor of at least blocks*256 elements."""
    if sink.dtype != torch.float32 or sink.numel() < blocks * 256 or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous float32 tensor of blocks*256 elements")
    check(lib().lt_probe_mfma_bf16(int(blocks), int(iters), _ptr(sink), _stream(stream)))
    return float(blocks) * 4 * iters * 8 * 16384


def lt_probe_read(buf: torch.Tensor, blocks: int, sink: torch.Tensor, stream=None) -> int:
    """Launch the read probe over all of buf; returns the bytes it reads."""
    nbytes = buf.numel() * buf.element_size()
    if not buf.is_contiguous() or sink.dtype != torch.int32 or sink.numel() < blocks:
        raise ValueError("buf must be contiguous; sink an int32 tensor of >= blocks elements")
    check(lib().lt_probe_read(_ptr(buf), nbytes, int(blocks), _ptr(sink), _stream(stream)))
    return nbytes
