"""LightTransfer-Test prefill over a stack of layers, through the C ABI.

For each layer in order (LightTransfer project page, Figure 2 caption;
Chinese write-up, "solution 2"):
  1. causal GQA prefill with LSE and the per-head lazy ratio (one call);
  2. the per-head ratios go to the host; the layer score is their mean;
  3. the score enters the lazy-layer queue; if the queue holds more than C
     layers, the highest-score layer leaves and its KV cache is compacted to
     the sink + recent rows and the full copy released (or, with eviction
     before the push, the highest of the C already queued leaves first).
The KV bytes held after each step (and while a layer's full KV is added,
before the queue's decision) are tracked by the library's queue
(lt_lazy_queue_kv_bytes), so the peak prefill KV can be checked against C
full layers + the rest streaming.

Run the 64-layer workload:  python -m kv_cache_compression_causal_amd.driver
Offline selection over P prompts:  python -m kv_cache_compression_causal_amd.driver --offline P
"""
from __future__ import annotations

import argparse
import json
import sys
import time
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Tuple

import numpy as np
import torch

from . import api, ops, synth
from ._lib import LT_BF16, LT_EVICT_AFTER_PUSH, LT_EVICT_BEFORE_PUSH, LT_F32


@dataclass
class DriverResult:
    layers: int
    capacity: int
    head_ratio: List[List[float]]           # [L][B*Hq] lazy ratio per (batch, head)
    layer_score: List[float]                # fp64 mean of each layer's ratios
    evicted_at_step: List[int]              # layer evicted after layer l's push, or -1
    is_streaming: List[int]                 # 1 for layers converted to streaming
    retained_bytes: List[int]               # KV bytes held after step l
    transient_bytes: List[int]              # KV bytes held at step l before the queue's pop
    full_bytes: int
    stream_bytes: int
    prefill_ms: List[float] = field(default_factory=list)
    wall_s: float = 0.0
    streaming_kv: Dict[int, Tuple[torch.Tensor, torch.Tensor]] = field(default_factory=dict)  # layer -> (k, v)


def run(layer_inputs: Callable[[int], Tuple[torch.Tensor, torch.Tensor, torch.Tensor]], layers: int,
        capacity: int, S: int, R: int, W: int, timing: bool = False,
        policy: int = LT_EVICT_AFTER_PUSH, emit: bool = False) -> DriverResult:
    """Run the layer stack.  ``layer_inputs(l)`` returns (q, k, v) for layer l
    on the device; the layer's k, v are its KV cache.  policy: the queue's
    eviction timing (LT_EVICT_AFTER_PUSH or LT_EVICT_BEFORE_PUSH).  With
    eviction before the push the victim does not depend on the current layer,
    so its KV counts as freed before the current layer's KV is stored.
    emit: every layer's prefill also writes its streaming slice
    (lt_prefill_attn_lse_lazy_emit); switching a layer then only releases its
    full KV (no compaction), and a layer at full size holds its slice too."""
    queue = api.LazyQueue(layers, capacity, policy)
    kv: Dict[int, Tuple[torch.Tensor, torch.Tensor]] = {}
    streaming_kv: Dict[int, Tuple[torch.Tensor, torch.Tensor]] = {}
    slices: Dict[int, Tuple[torch.Tensor, torch.Tensor]] = {}   # emitted, for layers still at full size
    head_ratio, scores, evicted, retained, transient, times = [], [], [], [], [], []
    is_stream = [0] * layers
    full_b = stream_b = 0
    out = lse = rows = None
    # Layer l's ratios go to the host through one of two pinned buffers,
    # copied on the stream right after its prefill; the host waits for them
    # (the per-layer device -> host sync) only after layer l + 1's prefill is
    # queued, which does not depend on the queue's decision, so the push and
    # the compaction of an evicted layer overlap that prefill.
    ratio_dev: List[Optional[torch.Tensor]] = [None, None]
    ratio_host: List[Optional[torch.Tensor]] = [None, None]
    ready: List[Optional[torch.cuda.Event]] = [None, None]
    pending = []   # (layer, slot, timing events) whose ratios are not read yet

    def finish(l: int, slot: int, ev_pair) -> None:
        ready[slot].synchronize()
        r = ratio_host[slot].numpy().copy()
        if ev_pair is not None:
            times.append(ev_pair[0].elapsed_time(ev_pair[1]))
        ev, score = queue.push_ratios(l, r)
        held_after, held_before = queue.kv_bytes()
        transient.append(held_before)
        retained.append(held_after)
        if ev >= 0:
            kf, vf = kv.pop(ev)
            if emit:
                streaming_kv[ev] = slices.pop(ev)   # written by its prefill: nothing to copy
            else:
                streaming_kv[ev] = ops.compact(kf, vf, S, R)
            del kf, vf   # the full KV of the evicted layer is released
            is_stream[ev] = 1
        head_ratio.append([float(x) for x in r])
        scores.append(score)
        evicted.append(ev)

    t_start = time.perf_counter()
    for l in range(layers):
        q, k, v = layer_inputs(l)
        B, Hq, N, D = q.shape
        Hkv = k.shape[1]
        if out is None or out.shape != q.shape or out.dtype != q.dtype:
            out = torch.empty_like(q)
            lse = torch.empty(B, Hq, N, device=q.device, dtype=torch.float32)
            rows = torch.empty(B, Hq, W, device=q.device, dtype=torch.float32)
            for i in range(2):
                ratio_dev[i] = torch.empty(B, Hq, device=q.device, dtype=torch.float32)
                ratio_host[i] = torch.empty(B * Hq, dtype=torch.float32, pin_memory=True)
                ready[i] = torch.cuda.Event()
        if l == 0:
            dt = LT_BF16 if q.dtype == torch.bfloat16 else LT_F32
            full_b, stream_b = api.lt_kv_bytes(B, Hkv, N, D, dt, S, R)
            queue.set_kv_bytes(full_b, stream_b, emit)
        slot = l % 2
        ratio = ratio_dev[slot]
        ev_pair = None
        if timing:
            ev_pair = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            ev_pair[0].record()
        if emit:
            n_slots = min(N, S + R)
            ks = torch.empty(B, Hkv, n_slots, D, device=q.device, dtype=q.dtype)
            vs = torch.empty_like(ks)
            api.lt_prefill_attn_lse_lazy_emit(q, k, v, out, lse, S, R, W, rows, ratio, ks, vs)
            slices[l] = (ks, vs)
        else:
            api.lt_prefill_attn_lse_lazy(q, k, v, out, lse, S, R, W, rows, ratio)
        if timing:
            ev_pair[1].record()
        ratio_host[slot].copy_(ratio.reshape(-1), non_blocking=True)
        ready[slot].record()
        kv[l] = (k, v)
        del q
        if pending:
            finish(*pending.pop())
        pending.append((l, slot, ev_pair))
    while pending:
        finish(*pending.pop())
    torch.cuda.synchronize()
    queue.close()
    return DriverResult(layers, capacity, head_ratio, scores, evicted, is_stream, retained, transient,
                        full_b, stream_b, times, time.perf_counter() - t_start, streaming_kv)


@dataclass
class OfflineResult:
    prompts: int
    layers: int
    capacity: int
    head_ratio: List[List[List[float]]]     # [P][L][B*Hq]
    prompt_score: List[List[float]]         # [P][L] fp64 mean of each layer's ratios on each prompt
    layer_score: List[float]                # [L] mean over prompts
    is_streaming: List[int]                 # offline selection
    test_time_streaming: List[List[int]]    # [P][L]: the queue's choice on each prompt alone
    prefill_ms: List[float] = field(default_factory=list)
    wall_s: float = 0.0


def offline(prompt_inputs: Callable[[int, int], Tuple[torch.Tensor, torch.Tensor, torch.Tensor]],
            prompts: int, layers: int, capacity: int, S: int, R: int, W: int,
            timing: bool = False) -> OfflineResult:
    """Offline selection (press-release page, "LightTransfer method"): run
    every prompt through every layer's prefill + lazy ratio (the same kernels
    as at test time), then lt_select_offline keeps the ``capacity`` layers
    with the lowest mean score full.  ``prompt_inputs(p, l)`` returns (q, k,
    v) of layer l on prompt p.  For comparison each prompt's test-time queue
    decision on its own ratios is reported too."""
    times: List[float] = []
    out = lse = rows = ratio_all = None
    t_start = time.perf_counter()
    for p in range(prompts):
        for l in range(layers):
            q, k, v = prompt_inputs(p, l)
            B, Hq, N, D = q.shape
            if out is None or out.shape != q.shape or out.dtype != q.dtype:
                out = torch.empty_like(q)
                lse = torch.empty(B, Hq, N, device=q.device, dtype=torch.float32)
                rows = torch.empty(B, Hq, W, device=q.device, dtype=torch.float32)
            if ratio_all is None:
                # every layer's ratios stay on the device until the last prefill:
                # no decision depends on them before the selection
                ratio_all = torch.empty(prompts, layers, B, Hq, device=q.device, dtype=torch.float32)
            if timing:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
            api.lt_prefill_attn_lse_lazy(q, k, v, out, lse, S, R, W, rows, ratio_all[p, l])
            if timing:
                e1.record()
                times.append((e0, e1))
            del q, k, v
    hr = ratio_all.reshape(prompts, layers, -1).cpu().numpy()   # [P, L, n] fp32
    times = [a.elapsed_time(b) for a, b in times]
    ratios = [[hr[p, l] for l in range(layers)] for p in range(prompts)]
    layer_score, st = api.lt_select_offline(hr, capacity)
    prompt_score, test_time = [], []
    for p in range(prompts):
        sc, _, st_p = api.lt_select_lazy_layers(hr[p], capacity)
        prompt_score.append([float(x) for x in sc])
        test_time.append([int(x) for x in st_p])
    return OfflineResult(prompts, layers, capacity, [[[float(x) for x in r] for r in pl] for pl in ratios],
                         prompt_score, [float(x) for x in layer_score], [int(x) for x in st], test_time,
                         times, time.perf_counter() - t_start)


def main(argv: Optional[List[str]] = None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--evict-before-push", action="store_true",
                    help="evict the laziest queued layer before pushing once the queue is full")
    ap.add_argument("--emit-slices", action="store_true",
                    help="each layer's prefill writes its streaming slice (no compaction on eviction)")
    ap.add_argument("--offline", type=int, default=0, metavar="P",
                    help="offline selection over P synthetic prompts instead of the test-time queue")
    args = ap.parse_args(argv)
    w = synth.DRIVER64
    L = args.layers or int(w.extra["layers"])
    C = int(w.extra["capacity"]) if args.layers is None else L // 2
    dev = torch.device("cuda:0")
    if args.offline > 0:
        print(f"[driver] offline selection: {args.offline} prompts x {L} layers, capacity {C}",
              file=sys.stderr, flush=True)

        def prompt_inputs(p, l):
            q, k, v, _, _ = synth.driver_layer(l, w, device=dev, prompt=p)
            return q, k, v

        off = offline(prompt_inputs, args.offline, L, C, w.S, w.R, w.W, timing=True)
        print(json.dumps({
            "workload": f"offline: {args.offline} prompts x {L} layers, B{w.B} N{w.N} Hq{w.Hq} Hkv{w.Hkv} "
                        f"D{w.D} bf16, S{w.S} R{w.R} W{w.W}, capacity {C}",
            "streaming_layers": [l for l in range(L) if off.is_streaming[l]],
            "layer_score": off.layer_score,
            "differs_from_test_time": [sum(a != b for a, b in zip(off.is_streaming, tt))
                                       for tt in off.test_time_streaming],
            "prefill_ms_mean": sum(off.prefill_ms) / len(off.prefill_ms),
            "wall_s": off.wall_s}), flush=True)
        return 0

    def inputs(l):
        q, k, v, _, _ = synth.driver_layer(l, w, device=dev)
        return q, k, v

    print(f"[driver] {L} layers of B{w.B} N{w.N} Hq{w.Hq} Hkv{w.Hkv} D{w.D}, capacity {C}",
          file=sys.stderr, flush=True)
    policy = LT_EVICT_BEFORE_PUSH if args.evict_before_push else LT_EVICT_AFTER_PUSH
    res = run(inputs, L, C, w.S, w.R, w.W, timing=True, policy=policy, emit=args.emit_slices)
    srt = sorted(res.layer_score)
    gaps = [b - a for a, b in zip(srt, srt[1:])]
    MiB = 1 << 20
    flop = 4.0 * w.B * w.Hq * w.D * w.N * (w.N + 1) / 2
    report = {
        "workload": f"driver64: {L} layers, B{w.B} N{w.N} Hq{w.Hq} Hkv{w.Hkv} D{w.D} bf16, "
                    f"S{w.S} R{w.R} W{w.W}, capacity {C}",
        "eviction": "before push" if args.evict_before_push else "after push",
        "streaming_slices": "written by each prefill" if args.emit_slices else "compacted on eviction",
        "streaming_layers": [l for l in range(L) if res.is_streaming[l]],
        "full_layers": [l for l in range(L) if not res.is_streaming[l]],
        "evicted_at_step": res.evicted_at_step,
        "layer_score": res.layer_score,
        "score_min": min(res.layer_score), "score_max": max(res.layer_score),
        "min_adjacent_score_gap": min(gaps) if gaps else None,
        "kv_all_full_MiB": L * res.full_bytes / MiB,
        "kv_retained_final_MiB": res.retained_bytes[-1] / MiB,
        "kv_peak_transient_MiB": max(res.transient_bytes) / MiB,
        "kv_reduction_pct": 100.0 * (1 - res.retained_bytes[-1] / (L * res.full_bytes)),
        "prefill_ms_mean": sum(res.prefill_ms) / len(res.prefill_ms),
        "prefill_tflops": flop / (sum(res.prefill_ms) / len(res.prefill_ms) * 1e-3) / 1e12,
        "wall_s": res.wall_s,
    }
    print(json.dumps(report), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
