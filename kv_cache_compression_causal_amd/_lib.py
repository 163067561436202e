"""ctypes loader for liblt.so: declares every exported symbol of include/lt.h
and include/lt_probe.h.

The library must exist (built by ``python -m kv_cache_compression_causal_amd.build``
or ``__graft_entry__.build()``); there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblt.so")
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblt_debug.so")

LT_OK, LT_ERR_NULL, LT_ERR_SHAPE, LT_ERR_DTYPE, LT_ERR_LAYOUT, LT_ERR_WORKSPACE, LT_ERR_HIP, \
    LT_ERR_VALUE = range(8)
LT_F32, LT_BF16 = 0, 1
LT_EVICT_AFTER_PUSH, LT_EVICT_BEFORE_PUSH = 0, 1

# Every symbol include/lt.h and include/lt_probe.h declare.
EXPORTS = (
    "lt_prefill_attn_lse_lazy", "lt_streaming_attn", "lt_hybrid_decode_workspace_bytes",
    "lt_hybrid_decode_attn", "lt_compact_kv_streaming", "lt_kv_bytes", "lt_lazy_queue_create",
    "lt_lazy_queue_push", "lt_lazy_queue_push_ratios", "lt_lazy_queue_destroy", "lt_select_lazy_layers", "lt_status_str",
    "lt_last_error", "lt_probe_mfma_bf16", "lt_probe_read", "lt_lazy_queue_create_policy",
    "lt_select_lazy_layers_policy", "lt_stream_cache_append", "lt_select_offline",
    "lt_prefill_attn_lse_lazy_varlen", "lt_streaming_attn_varlen", "lt_hybrid_decode_attn_varlen",
    "lt_compact_kv_streaming_varlen", "lt_stream_cache_append_varlen", "lt_prefill_attn_lse_lazy_emit",
    "lt_lazy_queue_set_kv_bytes", "lt_lazy_queue_kv_bytes", "lt_kv_accounting",
    "lt_hybrid_decode_attn_noalloc", "lt_hybrid_decode_attn_paged",
)
LT_DECODE_NOALLOC_SCRATCH_BYTES = 8 << 20


class LtView(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("sb", ctypes.c_int64), ("sh", ctypes.c_int64),
                ("sn", ctypes.c_int64)]


class LtShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("N", ctypes.c_int), ("Hq", ctypes.c_int),
                ("Hkv", ctypes.c_int), ("D", ctypes.c_int), ("dtype", ctypes.c_int),
                ("scale", ctypes.c_float)]


class LtError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load liblt.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def load_library(path: str) -> ctypes.CDLL:
    """Load a build of the library at `path` (liblt.so, or the LDS-poisoning
    liblt_debug.so the tests compare with it) with every signature declared."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m kv_cache_compression_causal_amd.build`")
    L = ctypes.CDLL(path)
    c_int, c_int64, c_void_p, c_size_t = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    fp = ctypes.POINTER(ctypes.c_float)
    L.lt_prefill_attn_lse_lazy.argtypes = [ctypes.POINTER(LtShape), LtView, LtView, LtView, LtView,
                                           c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p]
    L.lt_prefill_attn_lse_lazy.restype = c_int
    L.lt_streaming_attn.argtypes = [ctypes.POINTER(LtShape), LtView, LtView, LtView, LtView,
                                    c_void_p, c_int, c_int, c_void_p]
    L.lt_streaming_attn.restype = c_int
    L.lt_hybrid_decode_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int64,
                                                   ctypes.POINTER(c_size_t)]
    L.lt_hybrid_decode_workspace_bytes.restype = c_int
    L.lt_hybrid_decode_attn.argtypes = [c_int, c_int, c_int, c_int, c_int, ctypes.c_float, c_void_p,
                                        LtView, LtView, c_int64, c_void_p, c_void_p, c_void_p,
                                        c_size_t, c_void_p]
    L.lt_hybrid_decode_attn.restype = c_int
    L.lt_hybrid_decode_attn_noalloc.argtypes = [c_int, c_int, c_int, c_int, c_int, ctypes.c_float, c_void_p,
                                                LtView, LtView, c_int64, c_void_p, c_void_p, c_void_p]
    L.lt_hybrid_decode_attn_noalloc.restype = c_int
    L.lt_compact_kv_streaming.argtypes = [LtView, LtView, LtView, LtView, c_int, c_int, c_int,
                                          c_int, c_int, c_int, c_int, c_void_p]
    L.lt_compact_kv_streaming.restype = c_int
    L.lt_kv_bytes.argtypes = [c_int, c_int, c_int64, c_int, c_int, c_int, c_int,
                              ctypes.POINTER(c_int64), ctypes.POINTER(c_int64)]
    L.lt_kv_bytes.restype = c_int
    L.lt_lazy_queue_create.argtypes = [c_int, c_int, ctypes.POINTER(c_void_p)]
    L.lt_lazy_queue_create.restype = c_int
    L.lt_lazy_queue_push.argtypes = [c_void_p, c_int, ctypes.c_double, ctypes.POINTER(c_int)]
    L.lt_lazy_queue_push.restype = c_int
    L.lt_lazy_queue_push_ratios.argtypes = [c_void_p, c_int, fp, c_int, ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(c_int)]
    L.lt_lazy_queue_push_ratios.restype = c_int
    L.lt_lazy_queue_destroy.argtypes = [c_void_p]
    L.lt_lazy_queue_destroy.restype = None
    L.lt_select_lazy_layers.argtypes = [fp, c_int, c_int, c_int, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(c_int), ctypes.POINTER(ctypes.c_uint8)]
    L.lt_select_lazy_layers.restype = c_int
    L.lt_lazy_queue_create_policy.argtypes = [c_int, c_int, c_int, ctypes.POINTER(c_void_p)]
    L.lt_lazy_queue_create_policy.restype = c_int
    L.lt_select_lazy_layers_policy.argtypes = [fp, c_int, c_int, c_int, c_int,
                                               ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_int),
                                               ctypes.POINTER(ctypes.c_uint8)]
    L.lt_select_lazy_layers_policy.restype = c_int
    L.lt_stream_cache_append.argtypes = [LtView, LtView, c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                                         c_int, c_int, c_int64, c_void_p]
    L.lt_stream_cache_append.restype = c_int
    L.lt_select_offline.argtypes = [fp, c_int, c_int, c_int, c_int, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_uint8)]
    L.lt_select_offline.restype = c_int
    L.lt_prefill_attn_lse_lazy_varlen.argtypes = [ctypes.POINTER(LtShape), c_void_p, LtView, LtView, LtView,
                                                  LtView, c_void_p, c_int, c_int, c_int, c_void_p, c_void_p,
                                                  c_void_p]
    L.lt_prefill_attn_lse_lazy_varlen.restype = c_int
    L.lt_streaming_attn_varlen.argtypes = [ctypes.POINTER(LtShape), c_void_p, LtView, LtView, LtView, LtView,
                                           c_void_p, c_int, c_int, c_void_p]
    L.lt_streaming_attn_varlen.restype = c_int
    L.lt_prefill_attn_lse_lazy_emit.argtypes = [ctypes.POINTER(LtShape), c_void_p, LtView, LtView, LtView,
                                                LtView, c_void_p, c_int, c_int, c_int, c_void_p, c_void_p,
                                                LtView, LtView, c_void_p]
    L.lt_prefill_attn_lse_lazy_emit.restype = c_int
    L.lt_hybrid_decode_attn_varlen.argtypes = [c_int, c_int, c_int, c_int, c_int, ctypes.c_float, c_void_p,
                                               LtView, LtView, c_void_p, c_int64, c_void_p, c_void_p,
                                               c_void_p, c_size_t, c_void_p]
    L.lt_hybrid_decode_attn_varlen.restype = c_int
    L.lt_hybrid_decode_attn_paged.argtypes = [c_int, c_int, c_int, c_int, c_int, ctypes.c_float, c_void_p,
                                              LtView, LtView, c_int, c_int, c_void_p, c_int, c_void_p,
                                              c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    L.lt_hybrid_decode_attn_paged.restype = c_int
    L.lt_compact_kv_streaming_varlen.argtypes = [LtView, LtView, LtView, LtView, c_int, c_int, c_int, c_int,
                                                 c_int, c_int, c_int, c_void_p, c_void_p]
    L.lt_compact_kv_streaming_varlen.restype = c_int
    L.lt_stream_cache_append_varlen.argtypes = [LtView, LtView, c_void_p, c_void_p, c_int, c_int, c_int,
                                                c_int, c_int, c_int, c_void_p, c_void_p]
    L.lt_stream_cache_append_varlen.restype = c_int
    L.lt_lazy_queue_set_kv_bytes.argtypes = [c_void_p, c_int64, c_int64, c_int]
    L.lt_lazy_queue_set_kv_bytes.restype = c_int
    L.lt_lazy_queue_kv_bytes.argtypes = [c_void_p, ctypes.POINTER(c_int64), ctypes.POINTER(c_int64)]
    L.lt_lazy_queue_kv_bytes.restype = c_int
    L.lt_kv_accounting.argtypes = [ctypes.POINTER(c_int), c_int, c_int, c_int64, c_int64, c_int,
                                   ctypes.POINTER(c_int64), ctypes.POINTER(c_int64)]
    L.lt_kv_accounting.restype = c_int
    L.lt_status_str.argtypes = [c_int]
    L.lt_status_str.restype = ctypes.c_char_p
    L.lt_last_error.argtypes = []
    L.lt_last_error.restype = ctypes.c_char_p
    L.lt_probe_mfma_bf16.argtypes = [c_int, c_int, c_void_p, c_void_p]
    L.lt_probe_mfma_bf16.restype = c_int
    L.lt_probe_read.argtypes = [c_void_p, c_size_t, c_int, c_void_p, c_void_p]
    L.lt_probe_read.restype = c_int
    return L


def status_name(status: int) -> str:
    return lib().lt_status_str(status).decode()


def check(status: int) -> None:
    if status != LT_OK:
        raise LtError(status, lib().lt_last_error().decode())
