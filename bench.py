"""Benchmark of the LightTransfer-Test hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W]
                [--config {all,tiny,mistral8k,qwen32k,driver64,decode100k}]
                [--reps N] [--S S] [--R R] [--wobs W_obs] [--seed SEED]
                [--no-decode] [--no-driver] [--no-cpu] [--no-varlen]

Default (--config all): one JSON line whose headline is the qwen32k layer
(B1 N32768 Hq40 Hkv8 D128 bf16, keys of tokens 0..3 x3, S4 R1020 W128),
timed as a step of the method -- causal GQA prefill with LSE and the lazy
ratio + per-head mean, ratios to the host, layer score and queue push in the
library, and the KV of the evicted layer compacted to its sink + recent
slice; value = algorithmic prefill + lazy-numerator FLOP per step / wall
time per step.  Beside it, each workload of the pages' shapes:
  tiny        fp32 B1 N512 Hq4 Hkv1 D64, S4 R60 W32: launch latency (median
              of 100 launches, each timed by its own events) and the full
              oracle's time
  mistral8k   bf16 B1 N8192 Hq32 Hkv8 D128, S4 R1020 W64: prefill + lazy ratio,
              the plain prefill (the ratio's overhead, launches alternated)
              and streaming attention on the same tensors (medians of 20)
  qwen32k     the same three numbers at the headline shape, plus the prefill
              writing the layer's streaming slice, and a batch of four prompts
              (32K/24K/16K/8K tokens padded to 32K)
  decode100k  one hybrid decode step: B8, 100000-token context, 64 layers (32
              full, 32 streaming at S+R rows), one buffer per layer, the 64
              calls captured in a HIP graph; median of 20 replays; also with
              eight contexts from 100000 down to 12500 tokens
  driver64    the 64-layer LightTransfer-Test prefill with every layer's
              inputs resident in HBM: one timed pass (prefill, per-layer
              device->host sync, queue, compaction), the selection and the KV
              bytes; both eviction timings, slices written by the prefill,
              and offline selection over four prompts
--config X measures workload X alone and makes it the headline.  --S, --R,
--wobs and --seed replace those parameters in every workload measured.

roofline: the headline's dominant kernel, algorithmic FLOP (or bytes) per
launch over its mean duration from HIP events on the launch stream, against
the published peak.  cpu_baseline: the fp64 oracle on a bounded sample of
the same workload, on the host cores.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # MI355X dense bf16 matrix-core peak, FLOP/s
PEAK_HBM = 8.0e12       # MI355X HBM3E peak, B/s
PEAK_F32_VALU = 157.3e12  # MI355X fp32 vector peak, FLOP/s
METRIC = "prefill attn+lazy-ratio TFLOP/s @32K (% MFMA peak); hybrid decode HBM GB/s"
CONFIGS = ("all", "tiny", "mistral8k", "qwen32k", "driver64", "decode100k")


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


def median(xs):
    s = sorted(xs)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def traffic_from_profile(src_path: str, prof_path: str, key: str = "hbm_bytes_per_launch"):
    """HBM bytes per launch (or per step, with key) from a committed
    rocprofv3 --pmc summary, or None if the summary is missing or the kernel
    source changed since."""
    if not os.path.exists(prof_path):
        return None
    text = open(prof_path).read()
    sha = hashlib.sha256(open(src_path, "rb").read()).hexdigest()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(key + r":\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != sha:
        return None
    return float(m_b.group(1))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class Bench:
    """The legs of the benchmark; each returns a dict for the JSON line."""

    def __init__(self, args, torch, dev):
        self.args = args
        self.torch = torch
        self.dev = dev
        self.K = args.steps
        self.Wm = args.warmup
        self.reps = args.reps if args.reps is not None else args.steps  # timed launches of a per-launch leg
        self.stream = torch.cuda.current_stream()
        from kv_cache_compression_causal_amd import _lib, api, ops, synth
        self._lib, self.api, self.ops, self.synth = _lib, api, ops, synth

    # -- workloads with the command line's overrides ----------------------
    def workload(self, w):
        a = self.args
        kw = {}
        if a.S is not None:
            kw["S"] = a.S
        if a.R is not None:
            kw["R"] = a.R
        if a.wobs is not None and w.W > 0:
            kw["W"] = min(a.wobs, w.N)
        if a.seed is not None:
            kw["seed"] = a.seed
        return dataclasses.replace(w, **kw) if kw else w

    # -- timing -----------------------------------------------------------
    def events(self):
        E = self.torch.cuda.Event
        return E(enable_timing=True), E(enable_timing=True)

    def warm_clock(self, fn, seconds=0.3):
        """The chip raises its clock over the first milliseconds of load (a
        1 ms matrix-core run stays below the clock a 10 ms one holds): run fn
        untimed for about `seconds` before a leg's own warm-up."""
        t_end = time.perf_counter() + seconds
        n = 0
        while time.perf_counter() < t_end:
            for _ in range(8):
                fn()
            n += 8
            self.torch.cuda.synchronize()
        return n

    def time_each(self, fn, reps, warm=None):
        """Durations (ms) of `reps` launches of fn, each bracketed by its own
        events on the launch stream, after `warm` untimed ones."""
        for _ in range(self.Wm if warm is None else warm):
            fn()
        self.torch.cuda.synchronize()
        ev = []
        for _ in range(reps):
            a, b = self.events()
            a.record(self.stream)
            fn()
            b.record(self.stream)
            ev.append((a, b))
        self.torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    def paired(self, fa, fb, reps):
        """Two variants under the same clock: launches alternate (A B B A ...),
        each timed by its own events; returns the medians of A and B and the
        median over neighbouring pairs of the relative difference, so that a
        clock that drifts or dips weighs on both alike."""
        for _ in range(self.Wm):
            fa()
            fb()
        self.torch.cuda.synchronize()
        ev = []
        for r in range(reps):
            pair = {}
            for which in ((0, 1) if r % 2 == 0 else (1, 0)):
                a, b = self.events()
                a.record(self.stream)
                (fa if which == 0 else fb)()
                b.record(self.stream)
                pair[which] = (a, b)
            ev.append(pair)
        self.torch.cuda.synchronize()
        ta = [p[0][0].elapsed_time(p[0][1]) for p in ev]
        tb = [p[1][0].elapsed_time(p[1][1]) for p in ev]
        rel = [(y - x) / x for x, y in zip(ta, tb)]
        return median(ta), median(tb), 100.0 * median(rel)

    # -- the method's step at one layer (headline) -------------------------
    def step_leg(self, w, q, k, v):
        """K timed steps of one LightTransfer-Test layer: prefill + LSE + lazy
        ratio, ratios to the host through one of two pinned buffers, the
        layer's score and queue push in the library, and compaction of the
        evicted layer's KV.  A layer's push (and compaction) runs while the
        next layer's prefill is on the GPU: that prefill does not depend on
        the queue's decision, only the KV bookkeeping does."""
        torch, api = self.torch, self.api
        K, Wm, stream = self.K, self.Wm, self.stream
        B, N, Hq, Hkv, D, S, R, W = w.B, w.N, w.Hq, w.Hkv, w.D, w.S, w.R, w.W
        out = torch.empty_like(q)
        lse = torch.empty(B, Hq, N, device=self.dev, dtype=torch.float32)
        rows = torch.empty(B, Hq, W, device=self.dev, dtype=torch.float32)
        srows = min(N, S + R)
        k_st = torch.empty(B, Hkv, srows, D, device=self.dev, dtype=q.dtype)
        v_st = torch.empty_like(k_st)
        total_layers = K + Wm
        queue = api.LazyQueue(total_layers, total_layers // 2)
        ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
        ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
        layer = [0]
        ratio_d = [torch.empty(B, Hq, device=self.dev, dtype=torch.float32) for _ in range(2)]
        ratio_h = [torch.empty(B, Hq, dtype=torch.float32, pin_memory=True) for _ in range(2)]
        copied = [torch.cuda.Event() for _ in range(2)]
        pending = [None]

        def finish(slot):
            copied[slot].synchronize()  # the per-layer device->host hand-off of the method
            evicted, _ = queue.push_ratios(layer[0], ratio_h[slot].numpy())
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

        n_warm = self.warm_clock(lambda: api.lt_prefill_attn_lse_lazy(q, k, v, out, lse, S, R, W, rows,
                                                                       ratio_d[0], 0.0, stream))
        for i in range(Wm):
            step(i)
        drain()
        torch.cuda.synchronize()
        log(f"{w.name}: timing {K} steps after {n_warm + Wm} untimed prefill launches")
        t0 = time.perf_counter()
        for i in range(K):
            step(i, i)
        drain()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        queue.close()
        ms_step = (t1 - t0) * 1e3 / K
        kms = [a.elapsed_time(b) for a, b in zip(ev0, ev1)]
        fl = prefill_flop(B, Hq, N, D) + lazy_flop(B, Hq, N, D, S, R, W)
        return {"ms_per_step": ms_step, "value": fl / (ms_step * 1e-3) / 1e12, "flop": fl,
                "kernel_ms_mean": sum(kms) / len(kms), "kernel_ms_median": median(kms)}

    # -- one prefill workload: lazy ratio, its overhead, streaming ----------
    def prefill_leg(self, w, q, k, v, emit=False):
        torch, api = self.torch, self.api
        B, N, Hq, Hkv, D, S, R, W = w.B, w.N, w.Hq, w.Hkv, w.D, w.S, w.R, w.W
        out = torch.empty_like(q)
        lse = torch.empty(B, Hq, N, device=self.dev, dtype=torch.float32)
        rows = torch.empty(B, Hq, W, device=self.dev, dtype=torch.float32)
        ratio = torch.empty(B, Hq, device=self.dev, dtype=torch.float32)
        st = self.stream
        run_plain = lambda: api.lt_prefill_attn_lse_lazy(q, k, v, out, lse, S, R, 0, None, None, 0.0, st)
        run_lazy = lambda: api.lt_prefill_attn_lse_lazy(q, k, v, out, lse, S, R, W, rows, ratio, 0.0, st)
        self.warm_clock(run_lazy)
        plain_ms, lazy_ms, lazy_pct = self.paired(run_plain, run_lazy, self.reps)
        fl = prefill_flop(B, Hq, N, D) + lazy_flop(B, Hq, N, D, S, R, W)
        pfl = prefill_flop(B, Hq, N, D)
        res = {
            "prefill_lazy": {"ms_median": round(lazy_ms, 4), "tflops": round(fl / lazy_ms / 1e9, 2),
                             "frac_mfma_peak": round(fl / lazy_ms / 1e9 * 1e12 / PEAK_BF16, 4),
                             "flop_per_launch": fl},
            "prefill_plain": {"ms_median": round(plain_ms, 4), "tflops": round(pfl / plain_ms / 1e9, 2)},
            # launches alternated (A B B A ...): median over neighbouring pairs
            "lazy_overhead_pct": round(lazy_pct, 3),
        }
        log(f"{w.name}: prefill+lazy {lazy_ms:.3f} ms ({fl / lazy_ms / 1e9:.1f} TFLOP/s), plain {plain_ms:.3f} ms "
            f"({lazy_pct:+.2f}%)")
        if emit:
            srows = min(N, S + R)
            k_st = torch.empty(B, Hkv, srows, D, device=self.dev, dtype=q.dtype)
            v_st = torch.empty_like(k_st)
            run_emit = lambda: api.lt_prefill_attn_lse_lazy_emit(q, k, v, out, lse, S, R, W, rows, ratio, k_st,
                                                                 v_st, None, 0.0, st)
            base_ms, emit_ms, emit_pct = self.paired(run_lazy, run_emit, self.reps)
            res["prefill_emit"] = {"ms_median": round(emit_ms, 4), "ms_without_slice": round(base_ms, 4),
                                   "overhead_pct": round(emit_pct, 3),
                                   "what": "prefill+LSE+lazy ratio also writing the sink+recent KV slice "
                                           "(replaces the compaction kernel)"}
            log(f"{w.name}: writing the streaming slice {emit_pct:+.2f}%")
            del k_st, v_st
        sout = torch.empty_like(q)
        slse = torch.empty_like(lse)
        sts = self.time_each(lambda: api.lt_streaming_attn(q, k, v, sout, slse, S, R, 0.0, st), self.reps)
        st_ms = median(sts)
        sfl = streaming_flop(B, Hq, N, D, S, R)
        res["streaming"] = {"ms_median": round(st_ms, 4), "ms_mean": round(sum(sts) / len(sts), 4),
                            "tflops": round(sfl / st_ms / 1e9, 2),
                            "frac_mfma_peak": round(sfl / st_ms / 1e9 * 1e12 / PEAK_BF16, 4), "flop": sfl}
        log(f"{w.name}: streaming {st_ms:.3f} ms ({sfl / st_ms / 1e9:.1f} TFLOP/s)")
        return res

    # -- tiny fp32 layer ---------------------------------------------------
    def tiny_leg(self, cpu=True):
        torch, api = self.torch, self.api
        w = self.workload(self.synth.TINY)
        q, k, v = self.synth.workload_qkv(w, device=self.dev)
        B, N, Hq, D, S, R, W = w.B, w.N, w.Hq, w.D, w.S, w.R, w.W
        out = torch.empty_like(q)
        lse = torch.empty(B, Hq, N, device=self.dev, dtype=torch.float32)
        rows = torch.empty(B, Hq, W, device=self.dev, dtype=torch.float32)
        ratio = torch.empty(B, Hq, device=self.dev, dtype=torch.float32)
        ts = self.time_each(lambda: api.lt_prefill_attn_lse_lazy(q, k, v, out, lse, S, R, W, rows, ratio, 0.0,
                                                                 self.stream), 100, warm=10)
        fl = prefill_flop(B, Hq, N, D) + lazy_flop(B, Hq, N, D, S, R, W)
        ms = median(ts)
        res = {"workload": f"tiny: fp32 B{B} N{N} Hq{Hq} Hkv{w.Hkv} D{D}, S{S} R{R} W{W}, seed {w.seed}",
               "latency_us_median": round(ms * 1e3, 2), "latency_us_min": round(min(ts) * 1e3, 2),
               "reps": len(ts), "flop": fl, "tflops": round(fl / ms / 1e9, 4),
               "bound": "latency (a few workgroups; parity workload, no roofline fraction)"}
        log(f"tiny: {ms * 1e3:.1f} us per launch (median of {len(ts)})")
        if cpu:
            import oracle
            qh, kh, vh = (t.double().cpu().numpy() for t in (q, k, v))
            c0 = time.perf_counter()
            oracle.prefill(qh, kh, vh, S=S, R=R, W=W, streaming=True)
            t_cpu = time.perf_counter() - c0
            res["oracle_full_ms"] = round(t_cpu * 1e3, 3)
            res["oracle_threads"] = oracle.threads()
            res["oracle_what"] = "full fp64 oracle: out, LSE, streaming out/LSE, lazy rows and ratios"
        return res

    # -- variable-length prefill --------------------------------------------
    def varlen_leg(self):
        torch, api, synth = self.torch, self.api, self.synth
        vw, vlens = self.workload(synth.QWEN32K_VARLEN), synth.QWEN32K_VARLEN_LENS
        log("generating the variable-length batch")
        vq, vk, vv = synth.workload_qkv(vw, device=self.dev)
        vout = torch.empty_like(vq)
        vlse = torch.empty(vw.B, vw.Hq, vw.N, device=self.dev, dtype=torch.float32)
        vrows = torch.empty(vw.B, vw.Hq, vw.W, device=self.dev, dtype=torch.float32)
        vratio = torch.empty(vw.B, vw.Hq, device=self.dev, dtype=torch.float32)
        vlens_d = torch.tensor(vlens, device=self.dev, dtype=torch.int32)
        ts = self.time_each(lambda: api.lt_prefill_attn_lse_lazy_varlen(vq, vk, vv, vout, vlse, vlens_d, vw.S, vw.R,
                                                                        vw.W, vrows, vratio, 0.0, self.stream),
                            self.reps)
        v_ms = median(ts)
        v_fl = sum(prefill_flop(1, vw.Hq, n, vw.D) + lazy_flop(1, vw.Hq, n, vw.D, vw.S, vw.R, vw.W) for n in vlens)
        log(f"varlen prefill: {v_ms:.3f} ms, {v_fl / v_ms / 1e9:.1f} TFLOP/s")
        return {"workload": f"qwen32k-varlen: B4 prompts of {', '.join(map(str, vlens))} tokens padded to {vw.N}, "
                            f"Hq{vw.Hq} Hkv{vw.Hkv} D{vw.D} bf16, sink keys x3, S{vw.S} R{vw.R} W{vw.W}; "
                            "prefill+LSE+lazy ratio",
                "ms_median": round(v_ms, 4), "tflops": round(v_fl / v_ms / 1e9, 2),
                "frac_mfma_peak": round(v_fl / v_ms / 1e9 * 1e12 / PEAK_BF16, 4), "flop": v_fl}

    # -- hybrid decode -------------------------------------------------------
    def decode_leg(self, varlen=True):
        import numpy as np
        torch, api, ops, synth = self.torch, self.api, self.ops, self.synth
        dw = self.workload(synth.DECODE100K)
        L = int(dw.extra["layers"])
        nfull = int(dw.extra["full_layers"])
        log("allocating the 64-layer hybrid KV cache on device")
        qs, ks_, vs_, outs, lses, lens = [], [], [], [], [], []
        for l in range(L):
            ql, kl, vl = synth.decode_layer(l, dw, device=self.dev)
            qs.append(ql); ks_.append(kl); vs_.append(vl); lens.append(kl.shape[2])
            outs.append(torch.empty_like(ql))
            lses.append(torch.empty(dw.B, dw.Hq, device=self.dev, dtype=torch.float32))
        ws = ops.decode_workspace(dw.B, dw.Hq, dw.Hkv, dw.D, max(lens), self.dev)
        torch.cuda.synchronize()
        bytes_step = sum(2 * dw.B * dw.Hkv * n * dw.D * 2 + 2 * dw.B * dw.Hq * dw.D * 2 for n in lens)

        def decode_all(st):
            for l in range(L):
                api.lt_hybrid_decode_attn(qs[l], ks_[l], vs_[l], lens[l], outs[l], lses[l], ws, 0.0, st)

        cap = torch.cuda.Stream()

        def graph_of(fn):
            cap.wait_stream(self.stream)
            with torch.cuda.stream(cap):
                fn(cap)  # eager warm call on the capture stream
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                fn(cap)
            torch.cuda.synchronize()
            return g

        graph = graph_of(decode_all)
        log("decode graph captured")
        ts = self.time_each(graph.replay, self.reps, warm=3)
        d_ms = median(ts)
        gbps = bytes_step / (d_ms * 1e-3) / 1e9
        log(f"decode: {d_ms:.3f} ms/step, {gbps:.1f} GB/s")
        res = {"decode": {"workload": f"decode100k: B{dw.B}, context {dw.N}, {L} layers Hq{dw.Hq} Hkv{dw.Hkv} "
                                      f"D{dw.D} bf16, {nfull} full ({dw.N} rows) + {L - nfull} streaming "
                                      f"({lens[-1]} rows)",
                          "ms_per_step_median": round(d_ms, 4), "ms_per_step_mean": round(sum(ts) / len(ts), 4),
                          "gbps": round(gbps, 1), "frac_hbm_peak": round(gbps * 1e9 / PEAK_HBM, 4),
                          "bytes_per_step": bytes_step, "replays": len(ts)}}
        del graph
        if varlen:
            dlens = synth.DECODE100K_VARLEN_LENS
            full_lens = torch.tensor(dlens, device=self.dev, dtype=torch.int32)
            stream_lens = torch.tensor([min(n, lens[-1]) for n in dlens], device=self.dev, dtype=torch.int32)
            vbytes = sum(sum(2 * dw.Hkv * min(n, lens[l]) * dw.D * 2 for n in dlens) + 2 * dw.B * dw.Hq * dw.D * 2
                         for l in range(L))

            def decode_all_varlen(st):
                for l in range(L):
                    api.lt_hybrid_decode_attn_varlen(qs[l], ks_[l], vs_[l], full_lens if l < nfull else stream_lens,
                                                     lens[l], outs[l], lses[l], ws, 0.0, st)

            vgraph = graph_of(decode_all_varlen)
            vts = self.time_each(vgraph.replay, self.reps, warm=3)
            vd_ms = median(vts)
            vgbps = vbytes / (vd_ms * 1e-3) / 1e9
            log(f"varlen decode: {vd_ms:.3f} ms/step, {vgbps:.1f} GB/s")
            res["decode_varlen"] = {
                "workload": "decode100k-varlen: the decode100k step with contexts "
                            f"{dlens[0]}, {dlens[1]}, ..., {dlens[-1]} on the full layers (per-sequence lengths on "
                            f"the device), {lens[-1]} on the streaming ones",
                "ms_per_step_median": round(vd_ms, 4), "gbps": round(vgbps, 1),
                "frac_hbm_peak": round(vgbps * 1e9 / PEAK_HBM, 4), "bytes_per_step": vbytes}
            del vgraph
            # The same step over paged caches: every layer's [B, Hkv, rows, D]
            # cache read as a pool of PAGE-row pages (page b * Hkv * rows / PAGE
            # + c is rows [c * PAGE, (c + 1) * PAGE) of sequence b, the head
            # stride kept), and each sequence's pages listed in a shuffled
            # order: as many keys per sequence as the varlen step.  Pages of 32
            # rows take one table lookup per 32-key step, pages of 16 two.
            prng = np.random.default_rng(dw.seed)
            res["decode_paged"] = {
                "workload": "the decode100k-varlen step over paged caches, each sequence's pages in a shuffled "
                            "order of the pool (lt_hybrid_decode_attn_paged)", "bytes_per_step": vbytes}
            for PAGE in (32, 16):
                assert all(n % PAGE == 0 for n in lens)

                def pool_of(t, rows):
                    ppb = rows // PAGE
                    n_pages = (dw.B - 1) * dw.Hkv * ppb + ppb
                    return torch.as_strided(t, (n_pages, dw.Hkv, PAGE, dw.D), (PAGE * dw.D, rows * dw.D, dw.D, 1))

                def table_of(rows):
                    ppb = rows // PAGE
                    return torch.tensor(np.stack([b * dw.Hkv * ppb + prng.permutation(ppb) for b in range(dw.B)]),
                                        dtype=torch.int32, device=self.dev)

                tab_full, tab_stream = table_of(lens[0]), table_of(lens[-1])
                kpools = [pool_of(ks_[l], lens[l]) for l in range(L)]
                vpools = [pool_of(vs_[l], lens[l]) for l in range(L)]

                def decode_all_paged(st):
                    for l in range(L):
                        api.lt_hybrid_decode_attn_paged(qs[l], kpools[l], vpools[l],
                                                        tab_full if l < nfull else tab_stream,
                                                        full_lens if l < nfull else stream_lens, outs[l], lses[l],
                                                        ws, 0.0, st)

                pgraph = graph_of(decode_all_paged)
                pts = self.time_each(pgraph.replay, self.reps, warm=3)
                pd_ms = median(pts)
                pgbps = vbytes / (pd_ms * 1e-3) / 1e9
                log(f"paged decode, {PAGE}-row pages: {pd_ms:.3f} ms/step, {pgbps:.1f} GB/s")
                res["decode_paged"][f"page_{PAGE}"] = {
                    "ms_per_step_median": round(pd_ms, 4), "gbps": round(pgbps, 1),
                    "frac_hbm_peak": round(pgbps * 1e9 / PEAK_HBM, 4), "time_vs_varlen": round(pd_ms / vd_ms, 4)}
                del pgraph, kpools, vpools
        del qs, ks_, vs_, outs, lses, ws
        torch.cuda.empty_cache()
        return res

    # -- measured peaks ---------------------------------------------------------
    def probes_leg(self):
        torch, api = self.torch, self.api

        def best_ms(fn, reps=3):
            return min(self.time_each(fn, reps, warm=1))

        blocks, iters = 2048, 20000   # about 10 ms: long enough for the clock the chip holds under load
        psink = torch.empty(blocks * 256, device=self.dev, dtype=torch.float32)
        pfl = float(blocks) * 4 * iters * 8 * 16384
        mfma_ms = best_ms(lambda: api.lt_probe_mfma_bf16(blocks, iters, psink, self.stream))
        # the read probe over 16 GiB at several grid sizes: the best is the
        # read rate this machine delivers (a ceiling for the decode step)
        rbuf = torch.empty(16 << 30, device=self.dev, dtype=torch.uint8)
        read_by_grid = {}
        for blocks_r in (2048, 4096, 8192, 16384, 32768):
            rsink = torch.zeros(blocks_r, device=self.dev, dtype=torch.int32)
            ms = min(self.time_each(lambda: api.lt_probe_read(rbuf, blocks_r, rsink, self.stream), 2, warm=1))
            read_by_grid[blocks_r] = round(rbuf.numel() / (ms * 1e-3) / 1e9, 1)
        best_grid = max(read_by_grid, key=read_by_grid.get)
        res = {"mfma_bf16_tflops": round(pfl / (mfma_ms * 1e-3) / 1e12, 1),
               "hbm_read_gbps": read_by_grid[best_grid],
               "hbm_read_gbps_by_grid": read_by_grid,
               "spec_mfma_bf16_tflops": PEAK_BF16 / 1e12, "spec_hbm_gbps": PEAK_HBM / 1e9,
               "probes": "lt_probe_mfma_bf16: 2048 workgroups x 4 waves, 8 independent 16x16x32 bf16 MFMA chains "
                         "per wave on pseudo-random unit-size register operands, 20000 iterations, best of 3; "
                         "lt_probe_read: one pass of 16-byte nontemporal loads over 16 GiB (contiguous share per "
                         "workgroup, 16 loads in flight per lane), 2048-32768 workgroups, best of 2 each, the best "
                         "grid reported"}
        log(f"measured peaks: {res['mfma_bf16_tflops']} TFLOP/s bf16 MFMA, {res['hbm_read_gbps']} GB/s read")
        del rbuf, psink
        torch.cuda.empty_cache()
        return res

    # -- the 64-layer driver ------------------------------------------------------
    def driver_leg(self, offline=True, cpu=True):
        torch, synth = self.torch, self.synth
        from kv_cache_compression_causal_amd import driver
        dw = self.workload(synth.DRIVER64)
        L64, C = int(dw.extra["layers"]), int(dw.extra["capacity"])
        log(f"driver64: generating the {L64} layers' inputs in HBM")
        layers = []
        for l in range(L64):
            ql, kl, vl, _, _ = synth.driver_layer(l, dw, device=self.dev)
            layers.append((ql, kl, vl))
        torch.cuda.synchronize()
        layer_inputs = lambda l: layers[l]
        fl_layer = prefill_flop(dw.B, dw.Hq, dw.N, dw.D) + lazy_flop(dw.B, dw.Hq, dw.N, dw.D, dw.S, dw.R, dw.W)
        MiB = 1 << 20
        # one untimed pass like the timed one (its allocations of the evicted
        # layers' streaming caches fill torch's caching allocator, whose
        # first-time allocations otherwise stall the timed pass's host loop)
        # and the clock warm-up of the other prefill legs (generating 28 GiB of
        # inputs leaves the chip at a lower clock than a matrix-core load
        # holds), then the timed pass
        driver.run(layer_inputs, L64, C, dw.S, dw.R, dw.W)
        q0, k0, v0 = layers[0]
        o0 = torch.empty_like(q0)
        l0 = torch.empty(dw.B, dw.Hq, dw.N, device=self.dev, dtype=torch.float32)
        r0 = torch.empty(dw.B, dw.Hq, dw.W, device=self.dev, dtype=torch.float32)
        a0 = torch.empty(dw.B, dw.Hq, device=self.dev, dtype=torch.float32)
        self.warm_clock(lambda: self.api.lt_prefill_attn_lse_lazy(q0, k0, v0, o0, l0, dw.S, dw.R, dw.W, r0, a0, 0.0,
                                                                  self.stream))
        del o0, l0, r0, a0
        log("driver64: timed pass")
        res = driver.run(layer_inputs, L64, C, dw.S, dw.R, dw.W, timing=True)
        srt = sorted(res.layer_score)
        out = {
            "workload": f"driver64: {L64} layers of B{dw.B} N{dw.N} Hq{dw.Hq} Hkv{dw.Hkv} D{dw.D} bf16 (inputs "
                        f"resident in HBM), per-layer sink scale and recency bias, queue capacity {C}, "
                        f"S{dw.S} R{dw.R} W{dw.W}",
            "wall_s": round(res.wall_s, 4),
            "tflops_whole_pass": round(L64 * fl_layer / res.wall_s / 1e12, 2),
            "frac_mfma_peak_whole_pass": round(L64 * fl_layer / res.wall_s / PEAK_BF16, 4),
            "what_is_timed": "every layer's prefill+LSE+lazy ratio, its ratios to the host (a sync per layer, "
                             "waited for once the next layer's prefill is queued), the library's queue push and "
                             "the compaction of each evicted layer",
            "prefill_ms_mean": round(sum(res.prefill_ms) / len(res.prefill_ms), 4),
            "prefill_ms_median": round(median(res.prefill_ms), 4),
            "streaming_layers": [l for l in range(L64) if res.is_streaming[l]],
            "evicted_at_step": res.evicted_at_step,
            "score_min": min(res.layer_score), "score_max": max(res.layer_score),
            "min_adjacent_score_gap": min(b - a for a, b in zip(srt, srt[1:])) if L64 > 1 else None,
            "kv_all_full_MiB": L64 * res.full_bytes / MiB,
            "kv_retained_final_MiB": res.retained_bytes[-1] / MiB,
            "kv_peak_transient_MiB": max(res.transient_bytes) / MiB,
        }
        log(f"driver64: {res.wall_s:.3f} s whole pass ({out['tflops_whole_pass']} TFLOP/s), retained "
            f"{out['kv_retained_final_MiB']:.0f} MiB of {out['kv_all_full_MiB']:.0f}, "
            f"peak {out['kv_peak_transient_MiB']:.0f} MiB")
        gpu_ratio = {l: res.head_ratio[l] for l in (0, L64 - 1)}
        del res
        res_b = driver.run(layer_inputs, L64, C, dw.S, dw.R, dw.W, timing=True,
                           policy=self._lib.LT_EVICT_BEFORE_PUSH)
        out["evict_before_push"] = {
            "wall_s": round(res_b.wall_s, 4),
            "streaming_layers": [l for l in range(L64) if res_b.is_streaming[l]],
            "evicted_at_step": res_b.evicted_at_step,
            "kv_retained_final_MiB": res_b.retained_bytes[-1] / MiB,
            "kv_peak_transient_MiB": max(res_b.transient_bytes) / MiB,
        }
        del res_b
        res_e = driver.run(layer_inputs, L64, C, dw.S, dw.R, dw.W, timing=True, emit=True)
        base = out["evicted_at_step"]
        out["emitted_slices"] = {
            "wall_s": round(res_e.wall_s, 4),
            "same_selection": res_e.evicted_at_step == base,
            "compaction_launches": 0,
            "kv_retained_final_MiB": res_e.retained_bytes[-1] / MiB,
            "kv_peak_transient_MiB": max(res_e.transient_bytes) / MiB,
            "prefill_ms_mean": round(sum(res_e.prefill_ms) / len(res_e.prefill_ms), 4),
        }
        del res_e
        log(f"driver64: evict-before-push {out['evict_before_push']['wall_s']} s, emitted slices "
            f"{out['emitted_slices']['wall_s']} s")
        if cpu:
            out["oracle"] = self.driver_oracle(dw, layers, gpu_ratio, fl_layer)
        del layers
        torch.cuda.empty_cache()
        if offline:
            out_off = self.offline_leg(dw)
        else:
            out_off = None
        return out, out_off

    def driver_oracle(self, dw, layers, gpu_ratio, fl_layer):
        """The oracle on layers 0 and L-1 of the driver: every head's last W
        rows (what the lazy ratios and so the selection need), timed and
        extrapolated by FLOP to the whole 64-layer pass (x32 per layer)."""
        import numpy as np
        import oracle
        L64 = int(dw.extra["layers"])
        G = dw.Hq // dw.Hkv
        pos = np.arange(dw.N - dw.W, dw.N, dtype=np.int32)
        t_cpu, fl, err = 0.0, 0.0, 0.0
        for l in (0, L64 - 1):
            q, k, v = layers[l]
            for hk in range(dw.Hkv):
                kh = k[0, hk].double().cpu().numpy()
                vh = v[0, hk].double().cpu().numpy()
                for h in range(hk * G, (hk + 1) * G):
                    qr = q[0, h, dw.N - dw.W:].double().cpu().numpy()
                    c0 = time.perf_counter()
                    r = oracle.rows(kh, vh, pos, qr, S=dw.S, R=dw.R, lazy=True, streaming=False)
                    t_cpu += time.perf_counter() - c0
                    fl += sum(4.0 * dw.D * (int(p) + 1) + 2.0 * dw.D * min(dw.S + dw.R, int(p) + 1) for p in pos)
                    err = max(err, abs(float(r["lazy"].mean()) - gpu_ratio[l][h]))
        est = t_cpu * (L64 * fl_layer / (2 * fl))
        log(f"driver64 oracle: {t_cpu:.1f} s on the last W rows of layers 0 and {L64 - 1} "
            f"({fl / t_cpu / 1e9:.2f} GFLOP/s); whole-pass estimate {est / 3600:.1f} h")
        return {"layers": [0, L64 - 1], "sample": f"the last W={dw.W} rows of all {dw.Hq} heads of each layer "
                                                  f"(what the lazy ratios need), fp64",
                "seconds": round(t_cpu, 2), "gflops": round(fl / t_cpu / 1e9, 3),
                "whole_pass_estimate_s": round(est, 1),
                "whole_pass_estimate": "the measured FLOP rate applied to 64 full layers (x32 per measured layer)",
                "max_abs_ratio_diff_vs_gpu": err, "threads": oracle.threads()}

    def offline_leg(self, dw):
        torch, synth = self.torch, self.synth
        from kv_cache_compression_causal_amd import driver
        L64, C = int(dw.extra["layers"]), int(dw.extra["capacity"])
        P_off = 4
        log(f"running offline selection over {P_off} prompts")

        def prompt_inputs(p, l):
            ql, kl, vl, _, _ = synth.driver_layer(l, dw, device=self.dev, prompt=p)
            return ql, kl, vl

        off = driver.offline(prompt_inputs, P_off, L64, C, dw.S, dw.R, dw.W, timing=True)
        fl = prefill_flop(dw.B, dw.Hq, dw.N, dw.D) + lazy_flop(dw.B, dw.Hq, dw.N, dw.D, dw.S, dw.R, dw.W)
        med_ms = median(off.prefill_ms)
        res = {
            "workload": f"offline4: {P_off} synthetic prompts through the {L64} driver layers (per-layer sink "
                        f"scale and recency bias shared by all prompts), mean layer score over prompts, capacity {C}",
            "streaming_layers": [l for l in range(L64) if off.is_streaming[l]],
            "differs_from_test_time": [sum(a != b for a, b in zip(off.is_streaming, tt))
                                       for tt in off.test_time_streaming],
            "prefill_launches": len(off.prefill_ms),
            "prefill_ms_median": round(med_ms, 4),
            "prefill_tflops": round(fl / (med_ms * 1e-3) / 1e12, 2),
            "wall_s_with_input_generation": round(off.wall_s, 2),
        }
        log(f"offline4: {res['prefill_tflops']} TFLOP/s per launch, layers differing from each prompt's "
            f"test-time choice: {res['differs_from_test_time']}")
        del off
        torch.cuda.empty_cache()
        return res

    # -- the oracle on a row sample of a prefill workload ---------------------------
    def cpu_prefill(self, w, q, k, v, nrow):
        import numpy as np
        import oracle
        torch = self.torch
        log(f"timing the oracle on a {nrow}-row sample of {w.name}")
        B, N, Hq, Hkv, D, S, R, W = w.B, w.N, w.Hq, w.Hkv, w.D, w.S, w.R, w.W
        rng = np.random.default_rng(0)
        G = Hq // Hkv
        heads = rng.integers(0, Hq, size=nrow)
        pos = np.concatenate([np.arange(N - W, N), rng.integers(0, N, size=max(0, nrow - W))])[:nrow]
        kh_cache = {}
        flop, t_cpu = 0.0, 0.0
        for h in sorted(set(int(x) for x in heads)):
            sel = np.nonzero(heads == h)[0]
            hk = h // G
            if hk not in kh_cache:
                kh_cache[hk] = (k[0, hk].double().cpu().numpy(), v[0, hk].double().cpu().numpy())
            kh, vh = kh_cache[hk]
            ps = pos[sel].astype(np.int32)
            qr = q[0, h].index_select(0, torch.as_tensor(ps, device=self.dev, dtype=torch.long)).double().cpu().numpy()
            c0 = time.perf_counter()
            oracle.rows(kh, vh, ps, qr, S=S, R=R, lazy=True, streaming=False)
            t_cpu += time.perf_counter() - c0
            flop += sum(4.0 * D * (int(p) + 1) for p in ps)
            flop += sum(2.0 * D * min(S + R, int(p) + 1) for p in ps if p >= N - W)
        tf = flop / t_cpu / 1e12
        log(f"oracle: {tf * 1e3:.3f} GFLOP/s on {oracle.threads()} threads ({t_cpu:.1f} s)")
        return {"value": round(tf, 6), "unit": "TFLOP/s", "cores": oracle.threads(), "kind": "oracle",
                "cpu_model": cpu_model(),
                "sample": f"{nrow} query rows of the {w.name} layer (the last W={W} rows + uniform random rows, "
                          f"random heads), full softmax row materialised in fp64; {t_cpu:.1f} s; FLOP counted as "
                          f"for the GPU (4*D*(i+1) per row + lazy numerator)"}

    def cpu_decode(self):
        import oracle
        synth = self.synth
        dw = self.workload(synth.DECODE100K)
        nfull = int(dw.extra["full_layers"])
        t_layer, b_layer = {}, {}
        for l in (0, nfull):
            ql, kl, vl = synth.decode_layer(l, dw, device=self.dev)
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
        log(f"oracle decode: {b_step / t_step / 1e9:.3f} GB/s")
        return {"value": round(b_step / t_step / 1e9, 3), "unit": "GB/s", "cores": oracle.threads(),
                "kind": "oracle",
                "sample": f"decode100k layers 0 ({dw.N} rows) and {nfull} (S+R rows), batch element 0, fp64 "
                          f"({t_layer[0]:.2f} s + {t_layer[nfull]:.3f} s), extrapolated to the 64-layer step "
                          f"at B{dw.B}"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", choices=CONFIGS, default="all")
    ap.add_argument("--reps", type=int, default=None,
                    help="timed launches of each per-launch leg (default: --steps)")
    ap.add_argument("--S", type=int, default=None, help="sink keys (every workload measured)")
    ap.add_argument("--R", type=int, default=None, help="recent keys (every workload measured)")
    ap.add_argument("--wobs", type=int, default=None, help="observed last queries W (prefill workloads)")
    ap.add_argument("--seed", type=int, default=None, help="base seed of the synthetic inputs")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-driver", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=98304,
                    help="rows of the oracle's CPU sample of the headline prefill")
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

    import torch

    from kv_cache_compression_causal_amd import _lib, synth

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
    bench = Bench(args, torch, dev)
    cfg = args.config
    overrides = {k: getattr(args, k) for k in ("S", "R", "wobs", "seed") if getattr(args, k) is not None}
    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "data": "synthetic"}
    extra = {}

    def prefill_workload_leg(w, headline, emit):
        log(f"generating {w.name} inputs on device")
        q, k, v = synth.workload_qkv(w, device=dev)
        step = bench.step_leg(w, q, k, v) if headline else None
        legs = bench.prefill_leg(w, q, k, v, emit=emit)
        cpu = None
        if headline and not args.no_cpu:
            cpu = bench.cpu_prefill(w, q, k, v, args.cpu_rows if w.N >= 32768 else args.cpu_rows // 4)
        del q, k, v
        torch.cuda.empty_cache()
        return step, legs, cpu

    def step_fields(w, step, what):
        return {"value": round(step["value"], 2), "unit": "TFLOP/s", "ms_per_step": round(step["ms_per_step"], 4),
                "dtype": "bf16",
                "config": {"workload": f"{w.name} layer: B{w.B} N{w.N} Hq{w.Hq} Hkv{w.Hkv} D{w.D} bf16"
                                       f"{', sink keys x3' if w.sink_scale != 1.0 else ''}, S{w.S} R{w.R} W{w.W}, "
                                       f"seed {w.seed}; step = {what}",
                           "global_batch": w.B, "seq_len": w.N, "parallelism": "none (1 GPU)",
                           **({"overrides": overrides} if overrides else {})}}

    step_what = ("prefill+LSE+lazy ratio, ratio D2H, queue push (layer score in the library), KV compaction "
                 "(a layer's hand-off overlaps the next layer's prefill)")

    if cfg in ("all", "qwen32k", "mistral8k"):
        w = bench.workload(synth.QWEN32K if cfg != "mistral8k" else synth.MISTRAL8K)
        step, legs, cpu = prefill_workload_leg(w, True, emit=True)
        result.update(step_fields(w, step, step_what))
        achieved = step["flop"] / (step["kernel_ms_mean"] * 1e-3) / 1e12
        alt = legs["prefill_lazy"]
        # the headline workload's legs at the top level; the kernel time is
        # the mean over the timed steps' launches (the roofline's), the
        # median of the launches alternated with the plain prefill beside it
        legs["prefill_lazy"] = {"kernel_ms": round(step["kernel_ms_mean"], 4),
                                "kernel_ms_median": round(step["kernel_ms_median"], 4),
                                "tflops": round(achieved, 2), "frac_mfma_peak": round(achieved * 1e12 / PEAK_BF16, 4),
                                "flop_per_launch": step["flop"], "ms_median_alternated": alt["ms_median"],
                                "frac_mfma_peak_alternated": alt["frac_mfma_peak"]}
        result["headline_workload"] = w.name
        extra.update(legs)
        src = os.path.join(ROOT, "kv_cache_compression_causal_amd", "csrc", "attn_bf16.hip")
        traffic = traffic_from_profile(src, os.path.join(ROOT, "profiles", f"prefill_lazy_{w.name}_pmc.txt"))
        result["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16 / 1e12,
                              "unit": "TFLOP/s", "frac": round(achieved * 1e12 / PEAK_BF16, 4), "traffic": traffic,
                              "kernel": "attn_bf16_kernel<D=128, FULL_LAZY> + lazy_reduce_kernel",
                              "launches": args.steps,
                              "what": "algorithmic FLOP per launch / mean launch duration (HIP events on the launch "
                                      "stream, the timed steps)"}
        if cpu is not None:
            result["cpu_baseline"] = cpu
    if cfg == "all":
        extra["tiny"] = bench.tiny_leg(cpu=not args.no_cpu)
        w2 = bench.workload(synth.MISTRAL8K)
        _, legs2, _ = prefill_workload_leg(w2, False, emit=False)
        extra["mistral8k"] = legs2
        if not args.no_varlen:
            extra["qwen32k_varlen"] = bench.varlen_leg()
    if cfg == "tiny":
        t = bench.tiny_leg(cpu=not args.no_cpu)
        w = bench.workload(synth.TINY)
        extra["tiny"] = t
        ms = t["latency_us_median"] * 1e-3
        result.update({"value": t["tflops"], "unit": "TFLOP/s", "ms_per_step": round(ms, 5), "dtype": "f32",
                       "config": {"workload": t["workload"] + "; step = one prefill+LSE+lazy ratio launch "
                                                             "(median of 100, each timed by its own events)",
                                  "global_batch": w.B, "seq_len": w.N, "parallelism": "none (1 GPU)",
                                  **({"overrides": overrides} if overrides else {})}})
        result["roofline"] = {"bound": "alu", "achieved": t["tflops"], "peak": PEAK_F32_VALU / 1e12,
                              "unit": "TFLOP/s", "frac": round(t["tflops"] * 1e12 / PEAK_F32_VALU, 6),
                              "traffic": None, "kernel": "attn_f32_kernel<D=64, FULL_LAZY> + lazy_reduce_kernel",
                              "what": "latency-bound: a handful of workgroups"}
        if "oracle_full_ms" in t:
            result["cpu_baseline"] = {"value": round(t["flop"] / (t["oracle_full_ms"] * 1e-3) / 1e12, 6),
                                      "unit": "TFLOP/s", "cores": t["oracle_threads"], "kind": "oracle",
                                      "cpu_model": cpu_model(),
                                      "sample": "the whole tiny layer (full oracle, incl. streaming outputs)"}
    if cfg in ("all", "decode100k") and not args.no_decode:
        dres = bench.decode_leg(varlen=not args.no_varlen)
        extra.update(dres)
        if cfg == "decode100k":
            d = dres["decode"]
            result.update({"value": d["gbps"], "unit": "GB/s", "ms_per_step": d["ms_per_step_median"],
                           "dtype": "bf16",
                           "config": {"workload": d["workload"] + "; step = one decode token through the 64 layers "
                                                                  "(a replayed HIP graph), median of replays",
                                      "global_batch": 8, "seq_len": 100000, "parallelism": "none (1 GPU)",
                                      **({"overrides": overrides} if overrides else {})}})
            traffic = traffic_from_profile(os.path.join(ROOT, "kv_cache_compression_causal_amd", "csrc", "decode.hip"),
                                           os.path.join(ROOT, "profiles", "decode100k_pmc.txt"), "hbm_bytes_per_step")
            result["roofline"] = {"bound": "hbm", "achieved": d["gbps"], "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                                  "frac": d["frac_hbm_peak"], "traffic": traffic,
                                  "kernel": "decode_bf16_kernel<D=128> + decode_combine_kernel (64 layers)",
                                  "what": "algorithmic bytes per step / median step time of the replayed graph; "
                                          "traffic: FETCH_SIZE + WRITE_SIZE bytes of one step"}
            if not args.no_cpu:
                result["cpu_baseline"] = bench.cpu_decode()
        elif not args.no_cpu and "cpu_baseline" in result:
            result["cpu_baseline"]["decode"] = bench.cpu_decode()
    if cfg == "all":
        mp = bench.probes_leg()
        mp["prefill_lazy_frac_of_measured_mfma"] = round(result["roofline"]["achieved"] / mp["mfma_bf16_tflops"], 4)
        if "decode" in extra:
            mp["decode_frac_of_measured_read"] = round(extra["decode"]["gbps"] / mp["hbm_read_gbps"], 4)
        extra["measured_peaks"] = mp
    if cfg in ("all", "driver64") and not args.no_driver:
        drv, off = bench.driver_leg(offline=(cfg == "all"), cpu=not args.no_cpu)
        extra["driver64"] = drv
        if off is not None:
            extra["offline4"] = off
        if cfg == "driver64":
            w = bench.workload(synth.DRIVER64)
            result.update({"value": drv["tflops_whole_pass"], "unit": "TFLOP/s",
                           "ms_per_step": round(drv["wall_s"] * 1e3 / int(w.extra["layers"]), 4), "dtype": "bf16",
                           "config": {"workload": drv["workload"] + "; step = one layer of the timed 64-layer pass",
                                      "global_batch": w.B, "seq_len": w.N, "parallelism": "none (1 GPU)",
                                      **({"overrides": overrides} if overrides else {})}})
            result["roofline"] = {"bound": "mfma", "achieved": drv["tflops_whole_pass"],
                                  "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                                  "frac": drv["frac_mfma_peak_whole_pass"], "traffic": None,
                                  "kernel": "attn_bf16_kernel<D=128, FULL_LAZY> (64 launches) with the per-layer "
                                            "sync and queue"}
            if "oracle" in drv:
                o = drv["oracle"]
                result["cpu_baseline"] = {"value": round(o["gflops"] / 1e3, 6), "unit": "TFLOP/s",
                                          "cores": o["threads"], "kind": "oracle", "cpu_model": cpu_model(),
                                          "sample": o["sample"] + " of layers 0 and 63"}
    result.update(extra)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
