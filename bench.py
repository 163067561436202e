"""Benchmark of the LightTransfer-Test hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-driver] [--no-cpu] [--no-varlen]

Headline leg (the step): one LightTransfer-Test layer at the qwen32k shape
(B1 N32768 Hq40 Hkv8 D128 bf16, keys of tokens 0..3 x3, S4 R1020 W128):
causal GQA prefill with LSE and the lazy-ratio epilogue + per-head mean,
ratios to the host, layer score into the lazy-layer queue, and the KV of the
evicted layer compacted to its sink + recent slice.  value = algorithmic
prefill + lazy-numerator FLOP per step / wall time per step.

Other legs, reported beside it: the same prefill without the lazy ratio
(its overhead), streaming attention on the same tensors, one hybrid decode
step at B8 / 100000-token context over 64 layers (32 full, 32 streaming at
1024 rows; one distinct buffer per layer; the 64 calls are captured once in
a HIP graph and replayed), the 64-layer LightTransfer-Test prefill
(selected layers, eviction order, KV bytes) and offline selection over four
prompts, and variable-length batches: prefill over prompts of 32K/24K/16K/8K
tokens padded to 32K, and the decode step with eight contexts from 100000
down to 12500 tokens (lengths read per sequence on the device).

roofline: the prefill+lazy kernel, FLOP per launch over its mean duration
from HIP events on the launch stream, against the 2.5 PFLOP/s dense bf16
matrix-core peak.  cpu_baseline: the fp64 oracle on a bounded row sample of
the same workload, on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # MI355X dense bf16 matrix-core peak, FLOP/s
PEAK_HBM = 8.0e12       # MI355X HBM3E peak, B/s


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prefill_flop(B, Hq, N, D):
    return 4.0 * B * Hq * D * N * (N + 1) / 2


def lazy_flop(B, Hq, N, D, S, R, W):
    return 2.0 * B * Hq * D * sum(min(S + R, i + 1) for i in range(N - W, N))


def streaming_flop(B, Hq, N, D, S, R):
    K = S + R
    # sum_i min(i+1, K)
    tot = K * (K + 1) // 2 + max(0, N - K) * K if N >= K else N * (N + 1) // 2
    return 4.0 * B * Hq * D * tot


def traffic_from_profile(src_path: str, prof_path: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None
    if the summary is missing or the kernel source changed since."""
    if not os.path.exists(prof_path):
        return None
    text = open(prof_path).read()
    sha = hashlib.sha256(open(src_path, "rb").read()).hexdigest()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != sha:
        return None
    return float(m_b.group(1))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-driver", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=98304,
                    help="rows of the oracle's CPU sample")
    ap.add_argument("--copy-only", type=int, default=0, metavar="BYTES",
                    help="only run a device-to-device copy of BYTES, 5 times (the reference "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the kernels run on one GPU's share: the (batch, KV head) units a multi-GPU run "
              "would spread over its GPUs).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from kv_cache_compression_causal_amd import _lib, api, ops, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if not os.path.exists(_lib.LIB_PATH):
        from kv_cache_compression_causal_amd import build
        build.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_only:
        src = torch.empty(args.copy_only // 4, device=dev, dtype=torch.float32).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_only} bytes x5")
        return 0
    K, Wm = args.steps, args.warmup
    w = synth.QWEN32K
    B, N, Hq, Hkv, D, S, R, W = w.B, w.N, w.Hq, w.Hkv, w.D, w.S, w.R, w.W

    log(f"generating {w.name} inputs on device")
    q, k, v = synth.workload_qkv(w, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, N, device=dev, dtype=torch.float32)
    rows = torch.empty(B, Hq, W, device=dev, dtype=torch.float32)
    ratio = torch.empty(B, Hq, device=dev, dtype=torch.float32)
    srows = min(N, S + R)
    k_st = torch.empty(B, Hkv, srows, D, device=dev, dtype=q.dtype)
    v_st = torch.empty_like(k_st)
    sout = torch.empty_like(q)
    slse = torch.empty_like(lse)
    total_layers = K + Wm
    queue = api.LazyQueue(total_layers, total_layers // 2)
    stream = torch.cuda.current_stream()
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    layer = [0]
    # Each layer's ratios go to the host through one of two pinned buffers, so
    # that layer l's queue push (and the compaction it may trigger) runs while
    # layer l+1's prefill is on the GPU: the next prefill does not depend on
    # the queue's decision, only the KV bookkeeping does.
    ratio_d = [ratio, torch.empty_like(ratio)]
    ratio_h = [torch.empty(B, Hq, dtype=torch.float32, pin_memory=True) for _ in range(2)]
    copied = [torch.cuda.Event() for _ in range(2)]
    pending = [None]

    def finish(slot):
        copied[slot].synchronize()  # the per-layer device->host hand-off of the method
        score = float(ratio_h[slot].double().mean())
        evicted = queue.push(layer[0], score)
        layer[0] += 1
        if evicted >= 0:
            # one resident layer stands in for every layer: compact it
            api.lt_compact_kv_streaming(k, v, k_st, v_st, S, R, stream)

    def step(i, timed_idx=None):
        slot = i % 2
        if timed_idx is not None:
            ev0[timed_idx].record(stream)
        api.lt_prefill_attn_lse_lazy(q, k, v, out, lse, S, R, W, rows, ratio_d[slot], 0.0, stream)
        if timed_idx is not None:
            ev1[timed_idx].record(stream)
        ratio_h[slot].copy_(ratio_d[slot], non_blocking=True)
        copied[slot].record(stream)
        if pending[0] is not None:
            finish(pending[0])
        pending[0] = slot

    def drain():
        if pending[0] is not None:
            finish(pending[0])
            pending[0] = None

    log("warmup")
    for i in range(Wm):
        step(i)
    drain()
    torch.cuda.synchronize()
    log(f"timing {K} steps")
    t0 = time.perf_counter()
    for i in range(K):
        step(i, i)
    drain()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    kern_ms = sum(a.elapsed_time(b) for a, b in zip(ev0, ev1)) / K
    fl = prefill_flop(B, Hq, N, D) + lazy_flop(B, Hq, N, D, S, R, W)
    value = fl / (ms_step * 1e-3) / 1e12
    achieved = fl / (kern_ms * 1e-3) / 1e12
    log(f"prefill+lazy: {ms_step:.3f} ms/step, kernel {kern_ms:.3f} ms, {achieved:.1f} TFLOP/s")
    queue.close()

    # plain prefill (W = 0) for the lazy-ratio overhead
    def timed(fn, reps):
        for _ in range(Wm):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    # Two variants compared under the same clock: launches alternate between
    # them (A B B A ...), each timed by its own events, and the comparison is
    # the median over neighbouring pairs, so that a clock that drifts or dips
    # during the measurement weighs on both alike.
    def paired(fa, fb, reps):
        for _ in range(Wm):
            fa()
            fb()
        torch.cuda.synchronize()
        ev = []
        for r in range(reps):
            pair = {}
            for which in ((0, 1) if r % 2 == 0 else (1, 0)):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                (fa if which == 0 else fb)()
                b.record(stream)
                pair[which] = (a, b)
            ev.append(pair)
        torch.cuda.synchronize()
        ta = [p[0][0].elapsed_time(p[0][1]) for p in ev]
        tb = [p[1][0].elapsed_time(p[1][1]) for p in ev]
        rel = sorted((y - x) / x for x, y in zip(ta, tb))
        med = lambda xs: sorted(xs)[len(xs) // 2]
        return med(ta), med(tb), 100.0 * rel[len(rel) // 2]

    run_plain = lambda: api.lt_prefill_attn_lse_lazy(q, k, v, out, lse, S, R, 0, None, None, 0.0, stream)
    run_lazy = lambda: api.lt_prefill_attn_lse_lazy(q, k, v, out, lse, S, R, W, rows, ratio, 0.0, stream)
    # the same step writing the layer's streaming slice from the prefill itself
    run_emit = lambda: api.lt_prefill_attn_lse_lazy_emit(q, k, v, out, lse, S, R, W, rows, ratio, k_st, v_st,
                                                         None, 0.0, stream)
    plain_ms, lazy_ms, lazy_pct = paired(run_plain, run_lazy, K)
    log(f"plain prefill: {plain_ms:.3f} ms, with the lazy ratio: {lazy_ms:.3f} ms ({lazy_pct:+.2f}%)")
    lazy2_ms, emit_ms, emit_pct = paired(run_lazy, run_emit, K)
    log(f"prefill writing the streaming slice: {emit_ms:.3f} ms (without: {lazy2_ms:.3f} ms, {emit_pct:+.2f}%)")
    st_ms = timed(lambda: api.lt_streaming_attn(q, k, v, sout, slse, S, R, 0.0, stream), K)
    st_fl = streaming_flop(B, Hq, N, D, S, R)
    log(f"streaming: {st_ms:.3f} ms, {st_fl / st_ms / 1e9:.1f} TFLOP/s")

    result = {
        "metric": "prefill attn+lazy-ratio TFLOP/s @32K (% MFMA peak); hybrid decode HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen32k layer: B1 N32768 Hq40 Hkv8 D128 bf16, sink keys x3, "
                               "S4 R1020 W128; step = prefill+LSE+lazy ratio, ratio D2H, "
                               "queue push, KV compaction (a layer's hand-off overlaps the next "
                               "layer's prefill)",
                   "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)"},
        "prefill_lazy": {"kernel_ms": round(kern_ms, 4), "tflops": round(achieved, 2),
                         "frac_mfma_peak": round(achieved * 1e12 / PEAK_BF16, 4),
                         "flop_per_launch": fl},
        # with and without the lazy ratio, launches alternated (A B B A ...):
        # the median over neighbouring pairs of the relative difference
        "lazy_overhead_pct": round(lazy_pct, 3),
        "prefill_emit": {"ms": round(emit_ms, 4), "ms_without_slice": round(lazy2_ms, 4),
                         "overhead_pct": round(emit_pct, 3),
                         "what": "prefill+LSE+lazy ratio also writing the 4 MiB sink+recent KV slice "
                                 "(replaces the compaction kernel)"},
        "prefill_plain": {"ms": round(plain_ms, 4),
                          "tflops": round(prefill_flop(B, Hq, N, D) / plain_ms / 1e9, 2)},
        "streaming": {"ms": round(st_ms, 4), "tflops": round(st_fl / st_ms / 1e9, 2),
                      "flop": st_fl},
    }

    src = os.path.join(ROOT, "kv_cache_compression_causal_amd", "csrc", "attn_bf16.hip")
    traffic = traffic_from_profile(src, os.path.join(ROOT, "profiles", "prefill_lazy_qwen32k_pmc.txt"))
    result["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16 / 1e12,
                          "unit": "TFLOP/s", "frac": round(achieved * 1e12 / PEAK_BF16, 4),
                          "traffic": traffic,
                          "kernel": "attn_bf16_kernel<D=128, RB=3, BT=128, FULL_LAZY> + lazy_reduce_kernel"}
    del sout, slse

    # Variable-length batch: four prompts of 32K, 24K, 16K and 8K tokens padded to 32K.
    if not args.no_varlen:
        vw, vlens = synth.QWEN32K_VARLEN, synth.QWEN32K_VARLEN_LENS
        log("generating the variable-length batch")
        vq, vk, vv = synth.workload_qkv(vw, device=dev)
        vout = torch.empty_like(vq)
        vlse = torch.empty(vw.B, vw.Hq, vw.N, device=dev, dtype=torch.float32)
        vrows = torch.empty(vw.B, vw.Hq, vw.W, device=dev, dtype=torch.float32)
        vratio = torch.empty(vw.B, vw.Hq, device=dev, dtype=torch.float32)
        vlens_d = torch.tensor(vlens, device=dev, dtype=torch.int32)
        v_ms = timed(lambda: api.lt_prefill_attn_lse_lazy_varlen(vq, vk, vv, vout, vlse, vlens_d, vw.S, vw.R,
                                                                 vw.W, vrows, vratio, 0.0, stream), K)
        v_fl = sum(prefill_flop(1, vw.Hq, n, vw.D) + lazy_flop(1, vw.Hq, n, vw.D, vw.S, vw.R, vw.W)
                   for n in vlens)
        result["prefill_varlen"] = {
            "workload": "qwen32k-varlen: B4 prompts of 32768, 24576, 16384, 8192 tokens padded to 32768, "
                        "Hq40 Hkv8 D128 bf16, sink keys x3, S4 R1020 W128; prefill+LSE+lazy ratio",
            "ms": round(v_ms, 4), "tflops": round(v_fl / v_ms / 1e9, 2),
            "frac_mfma_peak": round(v_fl / v_ms / 1e9 * 1e12 / PEAK_BF16, 4), "flop": v_fl}
        log(f"varlen prefill: {v_ms:.3f} ms, {v_fl / v_ms / 1e9:.1f} TFLOP/s")
        del vq, vk, vv, vout, vlse, vrows, vratio
        torch.cuda.empty_cache()

    # hybrid decode step: B8, context 100000, 64 layers (32 full + 32 streaming)
    if not args.no_decode:
        dw = synth.DECODE100K
        L = int(dw.extra["layers"])
        nfull = int(dw.extra["full_layers"])
        log("allocating the 64-layer hybrid KV cache on device")
        qs, ks_, vs_, outs, lses, lens = [], [], [], [], [], []
        for l in range(L):
            ql, kl, vl = synth.decode_layer(l, dw, device=dev)
            qs.append(ql); ks_.append(kl); vs_.append(vl); lens.append(kl.shape[2])
            outs.append(torch.empty_like(ql))
            lses.append(torch.empty(dw.B, dw.Hq, device=dev, dtype=torch.float32))
        ws = ops.decode_workspace(dw.B, dw.Hq, dw.Hkv, dw.D, max(lens), dev)
        torch.cuda.synchronize()
        bytes_step = sum(2 * dw.B * dw.Hkv * n * dw.D * 2 + 2 * dw.B * dw.Hq * dw.D * 2 for n in lens)

        def decode_all(st):
            for l in range(L):
                api.lt_hybrid_decode_attn(qs[l], ks_[l], vs_[l], lens[l], outs[l], lses[l], ws, 0.0, st)

        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            decode_all(cap)  # eager warm call on the capture stream
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            decode_all(cap)
        torch.cuda.synchronize()
        log("decode graph captured")
        for _ in range(Wm):
            graph.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(K):
            graph.replay()
        b.record(stream)
        torch.cuda.synchronize()
        d_ms = a.elapsed_time(b) / K
        gbps = bytes_step / (d_ms * 1e-3) / 1e9
        log(f"decode: {d_ms:.3f} ms/step, {gbps:.1f} GB/s")
        result["decode"] = {"workload": "decode100k: B8, context 100000, 64 layers Hq40 Hkv8 D128 "
                                        "bf16, 32 full (100000 rows) + 32 streaming (1024 rows)",
                            "ms_per_step": round(d_ms, 4), "gbps": round(gbps, 1),
                            "frac_hbm_peak": round(gbps * 1e9 / PEAK_HBM, 4),
                            "bytes_per_step": bytes_step}
        del graph
        # The same step with eight different contexts on the full layers.
        if not args.no_varlen:
            dlens = synth.DECODE100K_VARLEN_LENS
            full_lens = torch.tensor(dlens, device=dev, dtype=torch.int32)
            stream_lens = torch.tensor([min(n, lens[-1]) for n in dlens], device=dev, dtype=torch.int32)
            vbytes = sum(sum(2 * dw.Hkv * min(n, lens[l]) * dw.D * 2 for n in dlens) + 2 * dw.B * dw.Hq * dw.D * 2
                         for l in range(L))

            def decode_all_varlen(st):
                for l in range(L):
                    api.lt_hybrid_decode_attn_varlen(qs[l], ks_[l], vs_[l], full_lens if l < nfull else stream_lens,
                                                     lens[l], outs[l], lses[l], ws, 0.0, st)

            with torch.cuda.stream(cap):
                decode_all_varlen(cap)
            torch.cuda.synchronize()
            vgraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(vgraph, stream=cap):
                decode_all_varlen(cap)
            torch.cuda.synchronize()
            for _ in range(Wm):
                vgraph.replay()
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(K):
                vgraph.replay()
            b.record(stream)
            torch.cuda.synchronize()
            vd_ms = a.elapsed_time(b) / K
            vgbps = vbytes / (vd_ms * 1e-3) / 1e9
            log(f"varlen decode: {vd_ms:.3f} ms/step, {vgbps:.1f} GB/s")
            result["decode_varlen"] = {
                "workload": "decode100k-varlen: the decode100k step with contexts 100000, 87500, ..., 12500 "
                            "on the full layers (per-sequence lengths on the device), 1024 on the streaming ones",
                "ms_per_step": round(vd_ms, 4), "gbps": round(vgbps, 1),
                "frac_hbm_peak": round(vgbps * 1e9 / PEAK_HBM, 4), "bytes_per_step": vbytes}
            del vgraph
        del qs, ks_, vs_, outs, lses, ws
        torch.cuda.empty_cache()

    # Measured peaks: the matrix-core and HBM-read rates the chip delivers in
    # practice (probe kernels of the library), next to the published peaks the
    # roofline fractions use.
    def best_ms(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    blocks, iters = 2048, 20000   # about 10 ms: long enough for the clock the chip holds under load
    psink = torch.empty(blocks * 256, device=dev, dtype=torch.float32)
    pfl = float(blocks) * 4 * iters * 8 * 16384
    mfma_ms = best_ms(lambda: api.lt_probe_mfma_bf16(blocks, iters, psink, stream))
    rbuf = torch.empty(4 << 30, device=dev, dtype=torch.uint8)
    rsink = torch.zeros(8192, device=dev, dtype=torch.int32)
    read_ms = best_ms(lambda: api.lt_probe_read(rbuf, 8192, rsink, stream))
    result["measured_peaks"] = {
        "mfma_bf16_tflops": round(pfl / (mfma_ms * 1e-3) / 1e12, 1),
        "hbm_read_gbps": round(rbuf.numel() / (read_ms * 1e-3) / 1e9, 1),
        "spec_mfma_bf16_tflops": PEAK_BF16 / 1e12, "spec_hbm_gbps": PEAK_HBM / 1e9,
        "probes": "lt_probe_mfma_bf16: 2048 workgroups x 4 waves, 8 independent 16x16x32 bf16 "
                  "MFMA chains per wave on pseudo-random unit-size register operands, 20000 iterations; "
                  "lt_probe_read: one pass of 16-byte nontemporal loads over 4 GiB (contiguous share per "
                  "workgroup), 8192 workgroups; best of 3"}
    mp = result["measured_peaks"]
    # the headline kernels against what this machine delivers, next to the spec fractions
    mp["prefill_lazy_frac_of_measured_mfma"] = round(achieved / mp["mfma_bf16_tflops"], 4)
    if "decode" in result:
        mp["decode_frac_of_measured_read"] = round(result["decode"]["gbps"] / mp["hbm_read_gbps"], 4)
    log(f"measured peaks: {result['measured_peaks']['mfma_bf16_tflops']} TFLOP/s bf16 MFMA, "
        f"{result['measured_peaks']['hbm_read_gbps']} GB/s read")
    del rbuf, rsink, psink
    torch.cuda.empty_cache()

    # The 64-layer LightTransfer-Test prefill: selection and KV bytes
    if not args.no_driver:
        from kv_cache_compression_causal_amd import driver
        dw = synth.DRIVER64
        log("running the 64-layer driver")

        def layer_inputs(l):
            ql, kl, vl, _, _ = synth.driver_layer(l, dw, device=dev)
            return ql, kl, vl

        res = driver.run(layer_inputs, int(dw.extra["layers"]), int(dw.extra["capacity"]), dw.S, dw.R,
                         dw.W, timing=True)
        srt = sorted(res.layer_score)
        MiB = 1 << 20
        L64 = res.layers
        result["driver64"] = {
            "workload": "driver64: 64 layers of the qwen32k shape, per-layer sink scale and recency "
                        "bias, queue capacity 32, S4 R1020 W128",
            "streaming_layers": [l for l in range(L64) if res.is_streaming[l]],
            "evicted_at_step": res.evicted_at_step,
            "kv_all_full_MiB": L64 * res.full_bytes / MiB,
            "kv_retained_final_MiB": res.retained_bytes[-1] / MiB,
            "kv_peak_transient_MiB": max(res.transient_bytes) / MiB,
            "min_adjacent_score_gap": min(b - a for a, b in zip(srt, srt[1:])),
            "prefill_ms_mean": round(sum(res.prefill_ms) / len(res.prefill_ms), 4),
        }
        log(f"driver64: retained {res.retained_bytes[-1] / MiB:.0f} MiB of {L64 * res.full_bytes / MiB:.0f}, "
            f"peak {max(res.transient_bytes) / MiB:.0f} MiB")
        torch.cuda.empty_cache()
        # The other eviction timing the pages describe: the laziest queued layer
        # leaves before the current one is stored.
        res_b = driver.run(layer_inputs, int(dw.extra["layers"]), int(dw.extra["capacity"]), dw.S, dw.R,
                           dw.W, timing=False, policy=_lib.LT_EVICT_BEFORE_PUSH)
        result["driver64"]["evict_before_push"] = {
            "streaming_layers": [l for l in range(L64) if res_b.is_streaming[l]],
            "evicted_at_step": res_b.evicted_at_step,
            "kv_retained_final_MiB": res_b.retained_bytes[-1] / MiB,
            "kv_peak_transient_MiB": max(res_b.transient_bytes) / MiB,
        }
        log(f"driver64 (evict before push): peak {max(res_b.transient_bytes) / MiB:.0f} MiB")
        del res_b
        torch.cuda.empty_cache()
        # Slices written by each layer's prefill: no compaction launches.
        res_e = driver.run(layer_inputs, int(dw.extra["layers"]), int(dw.extra["capacity"]), dw.S, dw.R,
                           dw.W, timing=True, emit=True)
        result["driver64"]["emitted_slices"] = {
            "same_selection": res_e.evicted_at_step == res.evicted_at_step,
            "compaction_launches": 0,
            "kv_retained_final_MiB": res_e.retained_bytes[-1] / MiB,
            "kv_peak_transient_MiB": max(res_e.transient_bytes) / MiB,
            "prefill_ms_mean": round(sum(res_e.prefill_ms) / len(res_e.prefill_ms), 4),
        }
        log(f"driver64 (emitted slices): peak {max(res_e.transient_bytes) / MiB:.0f} MiB")
        del res_e
        torch.cuda.empty_cache()
        # Offline selection: the same layers on several prompts, mean score, top half streaming.
        P_off = 4
        log(f"running offline selection over {P_off} prompts")

        def prompt_inputs(p, l):
            ql, kl, vl, _, _ = synth.driver_layer(l, dw, device=dev, prompt=p)
            return ql, kl, vl

        off = driver.offline(prompt_inputs, P_off, L64, int(dw.extra["capacity"]), dw.S, dw.R, dw.W,
                             timing=True)
        off_flop = prefill_flop(dw.B, dw.Hq, dw.N, dw.D) + lazy_flop(dw.B, dw.Hq, dw.N, dw.D, dw.S, dw.R,
                                                                    dw.W)
        mean_ms = sum(off.prefill_ms) / len(off.prefill_ms)
        result["offline4"] = {
            "workload": "offline4: 4 synthetic prompts through the 64 driver layers (per-layer sink scale "
                        "and recency bias shared by all prompts), mean layer score over prompts, capacity 32",
            "streaming_layers": [l for l in range(L64) if off.is_streaming[l]],
            "differs_from_test_time": [sum(a != b for a, b in zip(off.is_streaming, tt))
                                       for tt in off.test_time_streaming],
            "prefill_launches": len(off.prefill_ms),
            "prefill_ms_mean": round(mean_ms, 4),
            "prefill_tflops": round(off_flop / (mean_ms * 1e-3) / 1e12, 2),
            "wall_s": round(off.wall_s, 2),
        }
        log(f"offline4: {result['offline4']['prefill_tflops']} TFLOP/s per launch, layers differing from "
            f"each prompt's test-time choice: {result['offline4']['differs_from_test_time']}")
        del off
        torch.cuda.empty_cache()

    # CPU baseline: the oracle on a bounded row sample of the same workload
    if not args.no_cpu:
        import oracle
        log("timing the oracle on a row sample")
        nrow = args.cpu_rows
        rng = np.random.default_rng(0)
        G = Hq // Hkv
        heads = rng.integers(0, Hq, size=nrow)
        pos = np.concatenate([np.arange(N - W, N), rng.integers(0, N, size=nrow - W)])[:nrow]
        kh_cache = {}
        flop = 0.0
        t_cpu = 0.0
        for h in sorted(set(int(x) for x in heads)):
            sel = np.nonzero(heads == h)[0]
            hk = h // G
            if hk not in kh_cache:
                kh_cache[hk] = (k[0, hk].double().cpu().numpy(), v[0, hk].double().cpu().numpy())
            kh, vh = kh_cache[hk]
            ps = pos[sel].astype(np.int32)
            qr = q[0, h].index_select(0, torch.as_tensor(ps, device=dev, dtype=torch.long)).double().cpu().numpy()
            c0 = time.perf_counter()
            oracle.rows(kh, vh, ps, qr, S=S, R=R, lazy=True, streaming=False)
            t_cpu += time.perf_counter() - c0
            flop += sum(4.0 * D * (int(p) + 1) for p in ps)
            flop += sum(2.0 * D * min(S + R, int(p) + 1) for p in ps if p >= N - W)
        cpu_tflops = flop / t_cpu / 1e12
        cpu_model = "unknown"
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        cpu_model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        result["cpu_baseline"] = {"value": round(cpu_tflops, 6), "unit": "TFLOP/s",
                                  "cores": oracle.threads(), "kind": "oracle", "cpu_model": cpu_model,
                                  "sample": f"{nrow} query rows of the qwen32k layer (the last W=128 rows "
                                            f"+ uniform random rows, random heads), full softmax row "
                                            f"materialised in fp64; {t_cpu:.1f} s; FLOP counted as "
                                            f"for the GPU (4*D*(i+1) per row + lazy numerator)"}
        log(f"oracle: {cpu_tflops * 1e3:.3f} GFLOP/s on {oracle.threads()} threads ({t_cpu:.1f} s)")
        if not args.no_decode:
            # The oracle's decode: batch element 0 of one full and one streaming
            # layer of the decode step, extrapolated to the 64-layer step (x8
            # batch, x32 layers of each kind); bytes counted as for the GPU.
            dw = synth.DECODE100K
            nfull = int(dw.extra["full_layers"])
            t_layer, b_layer = {}, {}
            for l in (0, nfull):
                ql, kl, vl = synth.decode_layer(l, dw, device=dev)
                qh = ql[:1].double().cpu().numpy()
                kh = kl[:1].double().cpu().numpy()
                vh = vl[:1].double().cpu().numpy()
                del ql, kl, vl
                c0 = time.perf_counter()
                oracle.decode(qh, kh, vh)
                t_layer[l] = time.perf_counter() - c0
                b_layer[l] = 2 * dw.Hkv * kh.shape[2] * dw.D * 2 + 2 * dw.Hq * dw.D * 2
                del qh, kh, vh
            L = int(dw.extra["layers"])
            t_step = dw.B * (nfull * t_layer[0] + (L - nfull) * t_layer[nfull])
            b_step = dw.B * (nfull * b_layer[0] + (L - nfull) * b_layer[nfull])
            result["cpu_baseline"]["decode"] = {
                "value": round(b_step / t_step / 1e9, 3), "unit": "GB/s",
                "sample": f"decode100k layers 0 (100000 rows) and {nfull} (1024 rows), batch element 0, "
                          f"fp64 ({t_layer[0]:.2f} s + {t_layer[nfull]:.3f} s), extrapolated to "
                          f"the 64-layer step at B8"}
            log(f"oracle decode: {b_step / t_step / 1e9:.3f} GB/s")

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
