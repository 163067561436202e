"""Seeded synthetic inputs shaped like the LightTransfer workloads.

Holds no step of the method: only random tensors, the one place both the HIP
path and the oracle take their inputs from.  Values are drawn in fp32 from a
torch Philox generator seeded per tensor set (q, then k, then v), then
rounded to the working dtype (bf16 rounds to nearest even); the oracle sees
the same rounded values, upcast exactly.

Workloads (the pages name Qwen2.5-32B-Instruct, LLaMA and Mistral and
contexts up to 100K tokens; real prompts and weights are not used):
  tiny      fp32, B1 N512 Hq4 Hkv1 D64, seed 1, S4 R60 W32
  mistral8k bf16, B1 N8192 Hq32 Hkv8 D128, seed 2, S4 R1020 W64
  qwen32k   bf16, B1 N32768 Hq40 Hkv8 D128, seed 3, keys of tokens 0..3
            scaled by 3.0 (attention sinks), S4 R1020 W128
  driver64  64 layers of the qwen32k shape, layer l seeded 4000+l; sink keys
            scaled by s_l ~ U[0,4]; the last 1020 keys shifted by b_l ~ U[0,2]
            times the unit direction of the group's mean query; (s_l, b_l)
            from numpy default_rng(4); queue capacity 32
  offline4  4 prompts through the 64 driver layers: prompt p of layer l is
            seeded 4000+l+100000p, the layer's (s_l, b_l) shared by all
            prompts (prompt 0 is driver64 itself); capacity 32
  decode100k bf16, B8, context 100000, 64 layers of Hq40 Hkv8 D128, seed 5;
            layers 0..31 full (100000 rows), 32..63 streaming (1024 rows)
  qwen32k-varlen  four qwen32k prompts of 32768, 24576, 16384, 8192 tokens
            padded to 32768, seed 6, sink keys x3
  decode100k-varlen  the decode step with contexts 100000 * (8-b)/8 for
            sequence b on the full layers
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    dtype: torch.dtype
    seed: int
    S: int
    R: int
    W: int
    sink_scale: float = 1.0
    extra: Dict[str, float] = field(default_factory=dict)


TINY = Workload("tiny", 1, 512, 4, 1, 64, torch.float32, 1, 4, 60, 32)
MISTRAL8K = Workload("mistral8k", 1, 8192, 32, 8, 128, torch.bfloat16, 2, 4, 1020, 64)
QWEN32K = Workload("qwen32k", 1, 32768, 40, 8, 128, torch.bfloat16, 3, 4, 1020, 128, sink_scale=3.0)
DRIVER64 = Workload("driver64", 1, 32768, 40, 8, 128, torch.bfloat16, 4000, 4, 1020, 128,
                    extra={"layers": 64, "capacity": 32})
DECODE100K = Workload("decode100k", 8, 100000, 40, 8, 128, torch.bfloat16, 5, 4, 1020, 0,
                      extra={"layers": 64, "full_layers": 32})

# Variable-length batches (padded to the longest sequence): four qwen32k-shaped
# prompts of 32K, 24K, 16K and 8K tokens; and the decode step with eight
# contexts from 100000 down to 12500 tokens on the full layers.
QWEN32K_VARLEN = Workload("qwen32k-varlen", 4, 32768, 40, 8, 128, torch.bfloat16, 6, 4, 1020, 128,
                          sink_scale=3.0)
QWEN32K_VARLEN_LENS = (32768, 24576, 16384, 8192)
DECODE100K_VARLEN_LENS = tuple(100000 * (8 - b) // 8 for b in range(8))

WORKLOADS = {w.name: w for w in (TINY, MISTRAL8K, QWEN32K, DRIVER64, DECODE100K, QWEN32K_VARLEN)}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, seed: int, dtype=torch.float32, device="cpu",
           gen: Optional[torch.Generator] = None) -> torch.Tensor:
    """N(0,1) drawn in fp32 then rounded to ``dtype``."""
    g = gen if gen is not None else _gen(seed, device)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)


def qkv(B: int, N: int, Hq: int, Hkv: int, D: int, seed: int, dtype=torch.bfloat16,
        device="cpu", sink_tokens: int = 0, sink_scale: float = 1.0,
        spikes: Sequence[Tuple[int, float]] = ()
        ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """q [B,Hq,N,D], k/v [B,Hkv,N,D] ~ N(0,1) from one seeded generator.
    Keys of the first ``sink_tokens`` positions are multiplied by
    ``sink_scale`` in fp32 before rounding, and the key at each position p of
    ``spikes`` by its factor (scores against it then reach many times the
    spread of the others, in both signs)."""
    g = _gen(seed, device)
    q = torch.randn(B, Hq, N, D, generator=g, device=device, dtype=torch.float32)
    k = torch.randn(B, Hkv, N, D, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(B, Hkv, N, D, generator=g, device=device, dtype=torch.float32)
    if sink_tokens > 0 and sink_scale != 1.0:
        k[:, :, :sink_tokens, :] *= sink_scale
    for p, f in spikes:
        if 0 <= p < N:
            k[:, :, p, :] *= f
    return q.to(dtype), k.to(dtype), v.to(dtype)


def workload_qkv(w: Workload, device="cpu"):
    return qkv(w.B, w.N, w.Hq, w.Hkv, w.D, w.seed, w.dtype, device,
               sink_tokens=4 if w.sink_scale != 1.0 else 0, sink_scale=w.sink_scale)


def driver_layer_params(layers: int = 64, seed: int = 4) -> Tuple[np.ndarray, np.ndarray]:
    """(s_l, b_l) for the 64-layer driver: s ~ U[0,4], b ~ U[0,2]."""
    rng = np.random.default_rng(seed)
    s = rng.uniform(0.0, 4.0, size=layers)
    b = rng.uniform(0.0, 2.0, size=layers)
    return s, b


def driver_layer(l: int, w: Workload = DRIVER64, device="cpu", sink_tokens: int = 4,
                 recent: Optional[int] = None, prompt: int = 0):
    """Layer l of the 64-layer driver: q, k, v of the qwen32k shape, seed
    4000+l (+ 100000 * prompt for further prompts through the same layers);
    sink keys x s_l; keys of the last ``recent`` (default R) positions
    + b_l * unit(mean of the group's queries over positions and heads).
    (s_l, b_l) belong to the layer and are the same for every prompt."""
    s_all, b_all = driver_layer_params(int(w.extra.get("layers", 64)))
    s_l, b_l = float(s_all[l]), float(b_all[l])
    R = w.R if recent is None else recent
    g = _gen(w.seed + l + 100000 * prompt, device)
    q = torch.randn(w.B, w.Hq, w.N, w.D, generator=g, device=device, dtype=torch.float32)
    k = torch.randn(w.B, w.Hkv, w.N, w.D, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(w.B, w.Hkv, w.N, w.D, generator=g, device=device, dtype=torch.float32)
    G = w.Hq // w.Hkv
    k[:, :, :sink_tokens, :] *= s_l
    qm = q.view(w.B, w.Hkv, G, w.N, w.D).mean(dim=(2, 3))  # [B, Hkv, D]
    u = qm / qm.norm(dim=-1, keepdim=True)
    k[:, :, w.N - R:, :] += b_l * u[:, :, None, :]
    return q.to(w.dtype), k.to(w.dtype), v.to(w.dtype), s_l, b_l


def decode_layer(l: int, w: Workload = DECODE100K, device="cpu"):
    """Layer l of the decode step: q [B,Hq,D] and a cache [B,Hkv,rows,D] with
    rows = context for full layers (l < full_layers) and S+R otherwise."""
    full = int(w.extra.get("full_layers", 32))
    rows = w.N if l < full else min(w.N, w.S + w.R)
    g = _gen(w.seed * 1000 + l, device)
    q = torch.randn(w.B, w.Hq, w.D, generator=g, device=device, dtype=torch.float32).to(w.dtype)
    k = torch.randn(w.B, w.Hkv, rows, w.D, generator=g, device=device, dtype=torch.float32).to(w.dtype)
    v = torch.randn(w.B, w.Hkv, rows, w.D, generator=g, device=device, dtype=torch.float32).to(w.dtype)
    return q, k, v
