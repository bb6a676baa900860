#!/usr/bin/env python3
"""Benchmark of the MLA latent-KV insert / gather / pack path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = the long-context workload, end to end, on inputs already resident
in HBM:
  * grouped fp8 insert of 5 layers x 16384 tokens ([kv_c | k_pe] bf16 ->
    e4m3fn with per-layer scales) into five [4096, 64, 576] paged caches;
  * 16 chunks of 8192 context tokens (131072 in all) from a [4096, 64, 576]
    fp8 cache: latent gather (dequantised to bf16) then the fp8 full-key + V
    pack of that chunk's kv_b_proj output [8192, 64 heads, 128 + 128].
The metric is effective HBM bandwidth: the algorithmic bytes every kernel of a
step must read and write, divided by the step time.  The JSON line also
carries the roofline of the dominant kernel (the fp8 pack), the CPU oracle
timed on a bounded sample, and per-kernel figures of the other workloads
(small-batch insert latency, context epilogue, chunked-context pack).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
L, R, P, W = 5, 512, 64, 576


# ------------------------------------------------------------ byte counts --
def insert_bytes(layers, tokens, valid_rows=None, cache_elem=1):
    """Algorithmic bytes of one grouped insert: read bf16 kv_c + k_pe of every
    (layer, token), the slot of every (layer, token), the per-layer scale and
    cache pointer; write one cache entry per valid slot."""
    valid = layers * tokens if valid_rows is None else valid_rows
    return (layers * tokens * W * 2 + layers * tokens * 8 + layers * 12
            + valid * W * cache_elem)


def small_insert_bytes(valid_rows, slot_entries, layers, fp8):
    """Algorithmic bytes of a small-batch insert: only the rows that are
    written need their inputs read (a skipped token moves nothing); plus the
    slot entries, and for fp8 the per-layer scale and cache pointer.
    5 layers x 4 tokens with one -1 (fp8): 15 x (1152 + 576) + 32 + 20 + 40 =
    26,012 B; one layer x 16 tokens (bf16): 16 x (1152 + 1152) + 128 = 36,992 B."""
    return (valid_rows * W * 2 + valid_rows * W * (1 if fp8 else 2) + slot_entries * 8
            + (layers * 12 if fp8 else 0))


def gather_bytes(tokens, width=W):
    """Read one fp8 cache row and one slot per token; write a bf16 row."""
    return tokens * width + tokens * 8 + 4 + tokens * width * 2


def pack_fp8_bytes(tokens, heads, nope=128, rope=64, vdim=128):
    """Read the whole kv_b_proj output (k_nope and v halves) and k_pe once per
    token; write the fp8 key and the fp8 V."""
    return (tokens * heads * (nope + vdim) * 2 + tokens * rope * 2
            + tokens * heads * (nope + rope) + tokens * heads * vdim)


def gather_raw_bytes(tokens, width=W):
    """Read one fp8 cache row and one slot per token; write the same codes."""
    return tokens * width + tokens * 8 + tokens * width


def pack_fp8_kpe_raw_bytes(tokens, heads, nope=128, rope=64, vdim=128):
    """As the fp8 pack, with k_pe read as one byte per value."""
    return (tokens * heads * (nope + vdim) * 2 + tokens * rope
            + tokens * heads * (nope + rope) + tokens * heads * vdim)


def merge_bytes(tokens, heads, head_dim=128):
    """Read the accumulator and the chunk's partial (bf16 rows and fp32 lse);
    write the accumulator back."""
    return 3 * tokens * heads * head_dim * 2 + 3 * tokens * heads * 4


def new_token_bytes(tokens, heads, fp8, valid_rows, cache_elem=1, nope=128, rope=64, vdim=128):
    """Read the query [T, H, nope+rope], k_nope (and v in fp8 mode) from their
    strided views, the latent row [kv_c | k_pe], the position, the slot and
    the fp32 cos/sin row of each token; write the query and key rows (and fp8 V)
    and one cache entry per valid token."""
    ob = 1 if fp8 else 2
    per_row = (nope + rope) * 2 + nope * 2 + (vdim * 2 if fp8 else 0)
    per_row += 2 * (nope + rope) * ob + (vdim if fp8 else 0)
    per_tok = (R + P) * 2 + 8 + 8 + P * 4
    return tokens * heads * per_row + tokens * per_tok + valid_rows * W * cache_elem


def pack_bf16_bytes(tokens, heads, nope=128, rope=64):
    return tokens * heads * nope * 2 + tokens * rope * 2 + tokens * heads * (nope + rope) * 2


def epilogue_bytes(layers, tokens):
    """Read the [T, L, 576] projection output, slots, positions, gamma, the
    fp32 cos/sin rows of the positions used (the rotation's fast path reads
    only those; the low-order table words are read where it falls back);
    write one fp8 entry per row."""
    return (tokens * layers * W * 2 + layers * tokens * 8 + tokens * 8 + layers * R * 2
            + tokens * P * 4 + layers * 8 + layers * tokens * W)


# --------------------------------------------------------------- workload --
class LongContext:
    """Inputs of one step, generated on the device from fixed seeds."""

    def __init__(self, torch, mk, dev, num_tokens=16384, num_ctx=131072, chunk=8192, heads=64):
        from fp8_paged_insert_amd import synth

        self.torch, self.mk, self.dev = torch, mk, dev
        self.T, self.num_ctx, self.chunk, self.heads = num_tokens, num_ctx, chunk, heads
        g = synth.gen(5, dev)
        self.kv_c = synth.bf16_normal((L, num_tokens, R), g, dev)
        self.k_pe = synth.bf16_normal((L, num_tokens, P), g, dev)
        self.caches = [synth.random_bytes((4096, 64, W), g, dev) for _ in range(L)]
        self.scales = synth.f32_uniform((L,), 0.5, 2.0, g, dev)
        self.slots = torch.stack([synth.randperm(4096 * 64, g, dev)[:num_tokens]
                                  for _ in range(L)])
        self.ptrs = mk.cache_ptr_table(self.caches)
        c = synth.context_cache(dev, seed=55, num_blocks=4096, num_ctx=num_ctx)
        self.ctx_cache, self.src_slots = c["cache"], c["src_slots"]
        self.ctx_scale = torch.tensor([0.5], dtype=torch.float32, device=dev)
        g2 = synth.gen(56, dev)
        self.kvb = [synth.kv_b_proj_output(chunk, g2, dev, heads=heads)
                    for _ in range(num_ctx // chunk)]
        self.ws = torch.empty(chunk, W, dtype=torch.bfloat16, device=dev)
        self.ws2 = [torch.empty(chunk, W, dtype=torch.bfloat16, device=dev) for _ in range(2)]
        self.key = torch.empty(chunk, heads, 192, dtype=torch.uint8, device=dev)
        self.v8 = torch.empty(chunk, heads, 128, dtype=torch.uint8, device=dev)
        self.pack_windows = []

    # Timed steps record a pair of HIP events on the stream around their 15
    # back-to-back joint launches (one event before the first, one after the
    # last), so the window's length / 15 is the joint launch's average
    # duration, the gaps between the launches included.  Events recorded by
    # a launch itself around one joint launch read about 2.5 us longer than
    # the profiler's duration of that kernel.
    EVENT_EVERY = 1

    def arm_timing(self, steps):
        """Create the HIP events the timed windows will record into."""
        torch = self.torch
        n = (steps + self.EVENT_EVERY - 1) // self.EVENT_EVERY
        self.timed_steps = 0
        self.event_pool = []
        for _ in range(n):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            e1.record()
            self.event_pool.append((e0, e1))
        torch.cuda.synchronize()

    def bytes_per_step(self):
        n = self.num_ctx // self.chunk
        return (insert_bytes(L, self.T) + n * gather_bytes(self.chunk)
                + n * pack_fp8_bytes(self.chunk, self.heads))

    def step(self, time_pack=False, max_blocks=0):
        """One pass over the workload, in order on the current stream: the
        grouped insert, then the chunk loop with the joint launch -- gather of
        chunk 0, then for every chunk c the pack of c together with the gather
        of c + 1 into the other workspace (the last chunk packs alone).  With
        time_pack, every EVENT_EVERY-th step records a pair of events on the
        stream around its joint launches.  max_blocks > 0 caps the pack's grid
        (grid-stride loop)."""
        mk = self.mk
        mk.mla_kv_insert_grouped(self.kv_c, self.k_pe, self.ptrs, self.slots, 64, 64 * W, W,
                                 self.scales, "fp8")
        n = len(self.kvb)
        window = None
        if time_pack:
            if self.timed_steps % self.EVENT_EVERY == 0:
                window = self.event_pool.pop()
            self.timed_steps += 1
        mk.mla_ctx_latent_gather(self.ctx_cache, self.src_slots[:self.chunk], self.ws2[0],
                                 self.ctx_scale, "fp8")
        for c, kvb in enumerate(self.kvb):
            ws = self.ws2[c % 2]
            if c + 1 < n:
                if window is not None and c == 0:
                    window[0].record()
                nxt = self.src_slots[(c + 1) * self.chunk:(c + 2) * self.chunk]
                mk.mla_ctx_kv_pack_gather(kvb[..., :128], ws[:, 512:], self.key, self.ctx_cache,
                                          nxt, self.ws2[(c + 1) % 2], v=kvb[..., 128:],
                                          v_out=self.v8, mode=mk.MLA_PACK_KEY_V_FP8,
                                          cache_scale=self.ctx_scale, max_blocks=max_blocks)
                if window is not None and c == n - 2:
                    window[1].record()
                    self.pack_windows.append(window)
            else:
                mk.mla_ctx_kv_pack(kvb[..., :128], ws[:, 512:], self.key, v=kvb[..., 128:],
                                   v_out=self.v8, mode=mk.MLA_PACK_KEY_V_FP8,
                                   max_blocks=max_blocks)

    def step_separate(self):
        """The same work with the gather and the pack of every chunk as launches
        of their own."""
        mk = self.mk
        mk.mla_kv_insert_grouped(self.kv_c, self.k_pe, self.ptrs, self.slots, 64, 64 * W, W,
                                 self.scales, "fp8")
        for c, kvb in enumerate(self.kvb):
            mk.mla_ctx_latent_gather(self.ctx_cache,
                                     self.src_slots[c * self.chunk:(c + 1) * self.chunk],
                                     self.ws, self.ctx_scale, "fp8")
            mk.mla_ctx_kv_pack(kvb[..., :128], self.ws[:, 512:], self.key, v=kvb[..., 128:],
                               v_out=self.v8, mode=mk.MLA_PACK_KEY_V_FP8)


def time_kernel(torch, fn, reps=50, warmup=5):
    """Median device time (us) of fn() bracketed by events on the current stream."""
    for _ in range(warmup):
        fn()
    times = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    return statistics.median(times)


TRAFFIC = os.path.join(ROOT, "profiles", "pack_gather_long_context_hbm_traffic.json")


def sources_sha256(paths):
    import hashlib

    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per joint launch from the rocprofv3 counter runs recorded in
    profiles/, or None when the kernel's sources changed since they ran."""
    try:
        with open(TRAFFIC) as f:
            d = json.load(f)
        if sources_sha256(d["sources"]) != d["sources_sha256"]:
            return None
        return d["traffic_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def flush_llc(torch, buf):
    """Read 1 GiB: evicts the 256 MB last-level cache without leaving dirty
    lines for the next kernel to write back."""
    buf.view(torch.float32).sum()


# ------------------------------------------------------------- components --
def small_batch(torch, mk, dev):
    """Small-batch grouped fp8 insert (5 layers x 4 tokens, one -1 slot)."""
    import ctypes

    from fp8_paged_insert_amd import synth

    d = synth.small_batch_fp8(dev)
    caches = d["caches"]
    ptrs = mk.cache_ptr_table(caches)
    sm = d["slot_mapping"]
    kv, pe, sc = d["kv_c"], d["k_pe"], d["scales"]

    def call():
        mk.mla_kv_insert_grouped(kv, pe, ptrs, sm, 64, 64 * W, W, sc, "fp8")

    lib = mk.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    raw_args = (kv.data_ptr(), kv.stride(0), kv.stride(1), pe.data_ptr(), pe.stride(0),
                pe.stride(1), ptrs.data_ptr(), sc.data_ptr(), sm.data_ptr(), 0, L, 4, R, P, 64,
                64 * W, W, mk.MLA_KV_FP8_E4M3, stream)

    def raw():
        lib.mla_kv_insert_grouped(*raw_args)

    def per_call_us(fn, n=1000):
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n * 1e6

    plan = mk.prepare_insert_grouped(kv, pe, ptrs, sm, 64, 64 * W, W, sc, "fp8")
    wall_binding = per_call_us(call)
    wall_prepared = per_call_us(plan)
    wall_raw = per_call_us(raw)
    around_call = time_kernel(torch, raw, reps=200)
    # the kernel alone: events the launch itself records at its start and end
    ek0 = torch.cuda.Event(enable_timing=True)
    ek1 = torch.cuda.Event(enable_timing=True)
    ek0.record()
    ek1.record()
    torch.cuda.synchronize()
    kernel_times = []
    for _ in range(200):
        mk.set_launch_events(ek0, ek1)
        raw()
        ek1.synchronize()
        kernel_times.append(ek0.elapsed_time(ek1) * 1e3)
    kernel = statistics.median(kernel_times)
    # graph replay: 100 inserts captured once
    graph_us = None
    try:
        s = torch.cuda.Stream(dev)
        s.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(s):
            for _ in range(3):
                call()
        torch.cuda.current_stream(dev).wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(100):
                call()
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10):
            g.replay()
        torch.cuda.synchronize()
        graph_us = (time.perf_counter() - t0) / 1000 * 1e6
    except Exception as e:  # pragma: no cover - reported, not fatal
        graph_us = f"unavailable: {e}"
    # the same 20 rows as five single-layer launches
    per_layer = []
    for l in range(L):
        per_layer.append((kv[l:l + 1], pe[l:l + 1], mk.cache_ptr_table([caches[l]]),
                          sm[l].contiguous(), sc[l:l + 1]))

    def five():
        for a in per_layer:
            mk.mla_kv_insert_grouped(a[0], a[1], a[2], a[3], 64, 64 * W, W, a[4], "fp8")

    five_us = per_call_us(five, n=300)
    return {"workload": "grouped fp8 insert, 5 layers x 4 tokens (one -1 slot)",
            "us_per_launch_wall": round(wall_binding, 2),
            "us_per_launch_wall_prepared": round(wall_prepared, 2),
            "us_per_launch_wall_raw_abi": round(wall_raw, 2),
            "us_kernel": round(kernel, 2),
            "us_stream_events_around_call": round(around_call, 2),
            "us_per_launch_graph_replay": graph_us if isinstance(graph_us, str) else round(graph_us, 2),
            "us_five_single_layer_launches": round(five_us, 2),
            "target_us": 10.0,
            "bytes": small_insert_bytes(15, 4, L, True)}


def single_layer_component(torch, mk, dev):
    """Single-layer bf16 concat-and-cache (16 tokens into a [4, 16, 576]
    cache, no norm / rope): latency per launch, as for the small batch."""
    from fp8_paged_insert_amd import synth

    d = synth.single_layer_bf16(dev)
    cache = d["caches"][0]
    ptrs = mk.cache_ptr_table([cache])
    kv, pe, sm = d["kv_c"], d["k_pe"], d["slot_mapping"]
    T = kv.shape[1]
    lib = mk.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream
    raw_args = (kv.data_ptr(), kv.stride(0), kv.stride(1), pe.data_ptr(), pe.stride(0),
                pe.stride(1), ptrs.data_ptr(), None, sm.data_ptr(), 0, 1, T, R, P, 16,
                cache.stride(0), cache.stride(1), mk.MLA_KV_AUTO, stream)

    def call():
        mk.mla_kv_insert_grouped(kv, pe, ptrs, sm, 16, cache.stride(0), cache.stride(1), None,
                                 "auto")

    def raw():
        lib.mla_kv_insert_grouped(*raw_args)

    def per_call_us(fn, n=1000):
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n * 1e6

    ek0 = torch.cuda.Event(enable_timing=True)
    ek1 = torch.cuda.Event(enable_timing=True)
    ek0.record()
    ek1.record()
    torch.cuda.synchronize()
    kernel_times = []
    for _ in range(200):
        mk.set_launch_events(ek0, ek1)
        raw()
        ek1.synchronize()
        kernel_times.append(ek0.elapsed_time(ek1) * 1e3)
    return {"workload": "single-layer bf16 insert, 16 tokens into a [4,16,576] cache",
            "us_per_launch_wall": round(per_call_us(call), 2),
            "us_per_launch_wall_raw_abi": round(per_call_us(raw), 2),
            "us_kernel": round(statistics.median(kernel_times), 2),
            "bytes": small_insert_bytes(T, T, 1, False)}


def copy_ceiling(torch, mk, dev, flush):
    """Device-to-device copies as the ceiling the HBM-bound kernels are
    compared with: the runtime's copy (torch copy_, 1 GiB) and the library's
    streaming copy (the launch shape of its streaming kernels) at 1 GiB and
    at the total size of the long-context insert (142.2 MB moved), of the
    context epilogue (36.6 MB moved), of one gather (14.2 MB moved) and of the
    weight transpose (82.6 MB moved), and a streaming kernel with the fp8 pack's
    read:write mix (2:1) at the pack's size (437 MB moved); each timed by its own launch events after a
    cache flush (the runtime's copy with stream events), median of 20."""
    out = {}
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    times = []
    for i in range(23):
        flush_llc(torch, flush)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        if i >= 3:
            times.append(e0.elapsed_time(e1) * 1e3)
    us = statistics.median(times)
    out["runtime_copy_1GiB"] = {"bytes": 2 * n, "us": round(us, 2),
                                "GBps": round(2 * n / us / 1e3, 1),
                                "frac_of_peak": round(2 * n / us / 1e3 / HBM_PEAK_GBS, 4)}
    for name, moved in (("stream_copy_1GiB", 2 * n),
                        ("stream_copy_insert_size", insert_bytes(L, 16384)),
                        ("stream_copy_epilogue_size", epilogue_bytes(L, 4096)),
                        ("stream_copy_gather_size", gather_bytes(8192)),
                        ("stream_copy_weight_transpose_size", 2 * 7168 * L * W * 2)):
        half = (moved // 2) // 16 * 16
        us, p90 = kernel_us(torch, mk, lambda: mk.mla_stream_copy(dst[:half], src[:half]), flush,
                            reps=20, warm=3)
        out[name] = rate(us, p90, 2 * half)
    # the fp8 pack's read:write mix (two bytes read per byte written) at the
    # pack's size: the ceiling for the pack and the joint launch
    third = (pack_fp8_bytes(8192, 64) // 3) // 16 * 16
    us, p90 = kernel_us(torch, mk, lambda: mk.mla_stream_mix(dst[:third], src[:2 * third], 2),
                        flush, reps=20, warm=3)
    out["stream_mix_2to1_pack_size"] = rate(us, p90, 3 * third)
    del src, dst
    return out


def kernel_us(torch, mk, fn, flush, reps=100, warm=10):
    """Median and 90th-percentile duration of the one kernel fn launches,
    bracketed by events the kernel itself records (mla_set_launch_events),
    each launch after a cache flush (10 untimed launches first)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()            # torch creates the events on first record
    e1.record()
    torch.cuda.synchronize()
    times = []
    for i in range(reps + warm):
        flush_llc(torch, flush)
        mk.set_launch_events(e0, e1)
        fn()
        e1.synchronize()
        if i >= warm:
            times.append(e0.elapsed_time(e1) * 1e3)
    times.sort()
    return statistics.median(times), times[min(len(times) - 1, int(0.9 * len(times)))]


def rate(us, p90, nbytes):
    """Component line: median and p90 microseconds, bytes, median GB/s and
    fraction of the HBM peak."""
    return {"us": round(us, 2), "p90_us": round(p90, 2), "bytes": nbytes,
            "GBps": round(nbytes / us / 1e3, 1),
            "frac_of_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}


def context_pack_component(torch, mk, dev, flush):
    from fp8_paged_insert_amd import synth

    d = synth.context_pack(dev)
    ws = torch.empty(8192, W, dtype=torch.bfloat16, device=dev)
    ws8 = torch.empty(8192, W, dtype=torch.uint8, device=dev)
    sc = torch.tensor([0.5], device=dev)
    kvb = d["kvb"]
    kvh = synth.f16_normal((8192, 64, 256), synth.gen(44, dev), dev)
    key8 = torch.empty(8192, 64, 192, dtype=torch.uint8, device=dev)
    v8 = torch.empty(8192, 64, 128, dtype=torch.uint8, device=dev)
    keyb = torch.empty(8192, 64, 192, dtype=torch.bfloat16, device=dev)
    mk.mla_ctx_latent_gather(d["cache"], d["src_slots"], ws, sc, "fp8")
    mk.mla_ctx_latent_gather(d["cache"], d["src_slots"], ws8, None, "fp8")

    def gather():
        mk.mla_ctx_latent_gather(d["cache"], d["src_slots"], ws, sc, "fp8")

    def gather_raw():
        mk.mla_ctx_latent_gather(d["cache"], d["src_slots"], ws8, None, "fp8")

    def pack8():
        mk.mla_ctx_kv_pack(kvb[..., :128], ws[:, 512:], key8, v=kvb[..., 128:], v_out=v8,
                           mode=mk.MLA_PACK_KEY_V_FP8)

    def pack8_raw():
        mk.mla_ctx_kv_pack(kvb[..., :128], ws8[:, 512:], key8, v=kvb[..., 128:], v_out=v8,
                           mode=mk.MLA_PACK_KEY_V_FP8)

    def pack8_f16():
        mk.mla_ctx_kv_pack(kvh[..., :128], kvh[:, 0, 128:192], key8, v=kvh[..., 128:],
                           v_out=v8, mode=mk.MLA_PACK_KEY_V_FP8)

    def packb():
        mk.mla_ctx_kv_pack(kvb[..., :128], ws[:, 512:], keyb)

    # one GPU's share under 8-way tensor parallelism: heads 0..7 of the same
    # kv_b_proj output (a strided view), k_pe broadcast locally
    key8_tp = torch.empty(8192, 8, 192, dtype=torch.uint8, device=dev)
    v8_tp = torch.empty(8192, 8, 128, dtype=torch.uint8, device=dev)

    def pack8_tp8():
        mk.mla_ctx_kv_pack(kvb[:, :8, :128], ws[:, 512:], key8_tp, v=kvb[:, :8, 128:],
                           v_out=v8_tp, mode=mk.MLA_PACK_KEY_V_FP8)

    # the same fp8 pack as a grid-stride loop over capped grids of 16, 32 and
    # 64 workgroups of 256 threads per compute unit (about 10, 5 and 2.5
    # chunks per thread; the full grid has one)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    def pack8_capped(per_cu):
        return lambda: mk.mla_ctx_kv_pack(kvb[..., :128], ws[:, 512:], key8, v=kvb[..., 128:],
                                          v_out=v8, mode=mk.MLA_PACK_KEY_V_FP8,
                                          max_blocks=per_cu * cus)

    out = {"workload": "chunked-context pack, 8192 tokens x 64 heads (tp8 share: 8 heads)",
           "full_grid_blocks": (8192 * 64 * (12 + 8) + 255) // 256}
    for name, fn, nbytes in (("gather", gather, gather_bytes(8192)),
                             ("gather_raw_fp8", gather_raw, gather_raw_bytes(8192)),
                             ("pack_fp8", pack8, pack_fp8_bytes(8192, 64)),
                             ("pack_fp8_capped_16_per_cu", pack8_capped(16),
                              pack_fp8_bytes(8192, 64)),
                             ("pack_fp8_capped_32_per_cu", pack8_capped(32),
                              pack_fp8_bytes(8192, 64)),
                             ("pack_fp8_capped_64_per_cu", pack8_capped(64),
                              pack_fp8_bytes(8192, 64)),
                             ("pack_fp8_kpe_raw", pack8_raw, pack_fp8_kpe_raw_bytes(8192, 64)),
                             ("pack_fp8_fp16_inputs", pack8_f16, pack_fp8_bytes(8192, 64)),
                             ("pack_bf16", packb, pack_bf16_bytes(8192, 64)),
                             ("pack_fp8_tp8_share", pack8_tp8, pack_fp8_bytes(8192, 8))):
        us, p90 = kernel_us(torch, mk, fn, flush)
        out[name] = rate(us, p90, nbytes)
    return out


def epilogue_component(torch, mk, dev, flush):
    from fp8_paged_insert_amd import synth

    d = synth.context_epilogue(dev, with_gemm=False)
    T = d["num_tokens"]
    cs = torch.empty(T, 2 * P, dtype=torch.float32, device=dev)
    mk.mla_rope_cos_sin_cache(cs, T, P, 10000.0)
    ptrs = mk.cache_ptr_table(d["caches"])

    def epi():
        mk.mla_ctx_kv_epilogue(d["all_kv"], d["gamma"], d["eps"], d["positions"], cs, ptrs,
                               d["slot_mapping"], 64, 64 * W, W, d["scales"], "fp8")

    us, p90 = kernel_us(torch, mk, epi, flush)
    res = {"workload": "context-KV epilogue, 5 layers x 4096 tokens (norm+rope+fp8+scatter)",
           **rate(us, p90, epilogue_bytes(L, T))}
    return res


def cache_dtype_component(torch, mk, dev, flush):
    """The long-context insert (5 x 16384 rows) and the 8192-row gather with
    e4m3fn and with e5m2 caches, each launch timed on its own."""
    from fp8_paged_insert_amd import synth

    d = synth.long_context_insert(dev)
    L, T = d["num_layers"], d["num_tokens"]
    ptrs = mk.cache_ptr_table(d["caches"])
    pc = synth.context_pack(dev)
    ws = torch.empty(8192, W, dtype=torch.bfloat16, device=dev)
    sc = torch.tensor([0.5], device=dev)
    out = {"workload": "long-context insert 5 x 16384 rows into [4096,64,576] caches; "
                       "gather 8192 rows from a [512,64,576] cache"}
    for name in ("fp8_e4m3", "fp8_e5m2"):
        def ins():
            mk.mla_kv_insert_grouped(d["kv_c"], d["k_pe"], ptrs, d["slot_mapping"], 64, 64 * W, W,
                                     d["scales"], name)

        def gat():
            mk.mla_ctx_latent_gather(pc["cache"], pc["src_slots"], ws, sc, name)

        for kind, fn, nbytes in (("insert", ins, insert_bytes(L, T)),
                                 ("gather", gat, gather_bytes(8192))):
            us, p90 = kernel_us(torch, mk, fn, flush)
            out[f"{kind}_{name}"] = rate(us, p90, nbytes)
    return out


def merge_component(torch, mk, dev, flush):
    """One log-sum-exp merge of a chunk partial into the accumulator of the
    chunked-context loop: 16384 query tokens x 64 heads x 128 (bf16 rows,
    fp32 lse [heads, tokens])."""
    from fp8_paged_insert_amd import synth

    T, H, D = 16384, 64, 128
    d = synth.attention_partials(dev, num_tokens=T, heads=H, head_dim=D, chunks=2)
    acc, lacc = d["outs"][0].clone(), d["lses"][0].clone()
    part, plse = d["outs"][1], d["lses"][1]

    def merge():
        mk.mla_ctx_merge_chunk(acc, lacc, part, plse, mk.MLA_MERGE_ACCUMULATE)

    us, p90 = kernel_us(torch, mk, merge, flush)
    return {"workload": "merge of one chunk partial into the accumulator, 16384 tokens x 64 "
                        "heads x 128 (bf16 outputs, fp32 lse)",
            **rate(us, p90, merge_bytes(T, H, D))}


def new_token_component(torch, mk, dev, flush):
    """The new-token epilogue of one layer for an 8192-token prefill batch
    (8 requests continuing contexts of up to 4096 tokens) with 64 heads:
    RoPE of q_pe / k_pe, query and key rows (+ fp8 V), insert into a
    [512, 64, 576] e4m3fn cache; fp8 (e4m3fn) and bf16 attention inputs."""
    from fp8_paged_insert_amd import synth

    d = synth.new_tokens(dev)
    T, H = d["num_tokens"], d["num_heads"]
    cs = torch.empty(d["max_pos"], 2 * P, dtype=torch.float32, device=dev)
    mk.mla_rope_cos_sin_cache(cs, d["max_pos"], P, 10000.0)
    q, kvb, kv = d["q"], d["kvb"], d["kv"]
    valid = int((d["slots"] >= 0).sum())
    out = {"workload": "new-token epilogue, 8192 tokens x 64 heads, one layer, "
                       "e4m3fn cache [512, 64, 576]"}
    # fp8: a plain cast of the query / key / V (no scales, as the chunked
    # pack's op); fp8_scaled: with per-tensor q / k / v scales (exact x / scale)
    for name, fp8, scaled in (("fp8", True, False), ("fp8_scaled", True, True),
                              ("bf16", False, False)):
        odt = torch.uint8 if fp8 else torch.bfloat16
        qo = torch.empty(T, H, 192, dtype=odt, device=dev)
        ko = torch.empty(T, H, 192, dtype=odt, device=dev)
        kw = dict(v=kvb[:, :, 128:], v_out=torch.empty(T, H, 128, dtype=torch.uint8, device=dev),
                  mode=mk.MLA_PACK_KEY_V_FP8) if fp8 else {}
        if scaled:
            kw.update(q_scale=d["q_scale"], k_scale=d["k_scale"], v_scale=d["v_scale"])
        cache = d["cache"]

        def run():
            mk.mla_new_token_epilogue(q[:, :, :128], q[:, :, 128:], kvb[:, :, :128], kv[:, :R],
                                      kv[:, R:], d["positions"], cs, qo, ko, cache=cache,
                                      slot_mapping=d["slots"], kv_cache_dtype="fp8",
                                      cache_scale=d["cache_scale"], **kw)

        us, p90 = kernel_us(torch, mk, run, flush)
        out[name] = rate(us, p90, new_token_bytes(T, H, fp8, valid))
    return out


def projection_component(torch, mk, dev, flush):
    from fp8_paged_insert_amd import synth

    g = synth.gen(3, dev)
    x = synth.bf16_normal((4096, 7168), g, dev)
    # the weight as the workload states it, the [K, N] matrix, converted
    # into the [N, K] storage the projection reads by the library's transpose
    w_kn = synth.bf16_normal((7168, L * W), g, dev, std=0.02)
    w_nk = torch.empty(L * W, 7168, dtype=torch.bfloat16, device=dev)
    mk.mla_transpose_bf16(w_kn, w_nk)
    tr_us, tr_p90 = kernel_us(torch, mk, lambda: mk.mla_transpose_bf16(w_kn, w_nk), flush)
    y = torch.empty(4096, L * W, dtype=torch.bfloat16, device=dev)
    try:
        us, p90 = kernel_us(torch, mk, lambda: mk.mla_ctx_kv_proj(x, w_nk, y), flush)
    except mk.MlaError as e:
        return {"workload": "context_kv_proj 4096x7168 . 7168x2880", "status": str(e)}
    # the vendor library GEMM on the same operands, for context (torch.matmul
    # -> hipBLASLt), timed with stream events around the call after the same flush
    ref = []
    for i in range(25):
        flush_llc(torch, flush)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.matmul(x, w_nk.t())
        e1.record()
        e1.synchronize()
        if i >= 3:
            ref.append(e0.elapsed_time(e1) * 1e3)
    # end to end: the projection, then the epilogue reading its output as
    # [T, L, 576] and inserting into 5 fp8 caches (stream events around both)
    e = synth.context_epilogue(dev, with_gemm=False)
    cs = torch.empty(4096, 2 * P, dtype=torch.float32, device=dev)
    mk.mla_rope_cos_sin_cache(cs, 4096, P, 10000.0)
    ptrs = mk.cache_ptr_table(e["caches"])
    e2e, e2e_tr = [], []
    for i in range(25):
        for with_tr, acc in ((False, e2e), (True, e2e_tr)):
            flush_llc(torch, flush)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            if with_tr:
                mk.mla_transpose_bf16(w_kn, w_nk)
            mk.mla_ctx_kv_proj(x, w_nk, y)
            mk.mla_ctx_kv_epilogue(y.view(4096, L, W), e["gamma"], e["eps"], e["positions"], cs,
                                   ptrs, e["slot_mapping"], 64, 64 * W, W, e["scales"], "fp8")
            e1.record()
            e1.synchronize()
            if i >= 3:
                acc.append(e0.elapsed_time(e1) * 1e3)
    flops = 2 * 4096 * 7168 * L * W
    # the matrix cores' own ceiling on this machine: the issue interval of
    # v_mfma_f32_32x32x16_bf16 and the clock held under full MFMA load, read
    # by the library's rate probe (one workgroup of 4 wavefronts per CU)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    clocks = torch.zeros(16 * cus, dtype=torch.int64, device=dev)
    iters = 4096
    mk.mla_mfma_rate(clocks, iters)  # warm-up
    mk.mla_mfma_rate(clocks, iters)
    torch.cuda.synchronize()
    c = clocks.view(-1, 4).cpu()
    cyc = (c[:, 1] - c[:, 0]).double()
    per_mfma = float(cyc.mean()) / (iters * 12)
    ghz = float(cyc.sum() / (c[:, 3] - c[:, 2]).double().sum()) * 0.1
    mfma_flops = 2 * 32 * 32 * 16
    # per wavefront of the projection: 4 x 3 tiles of 32 x 32, K / 16 steps
    proj_mfmas = 12 * 7168 // 16
    ceiling = {"cycles_per_mfma_32x32x16_bf16": round(per_mfma, 2),
               "sustained_clock_ghz": round(ghz, 3),
               "tflops_at_sustained_clock": round(4 * cus * mfma_flops / per_mfma * ghz / 1e3, 1),
               "tflops_at_2_4_ghz": round(4 * cus * mfma_flops / per_mfma * 2.4 / 1e3, 1),
               "projection_mfma_bound_us": round(proj_mfmas * per_mfma / ghz / 1e3, 2),
               "note": "the projection's MFMAs alone at this issue interval and clock "
                       "(240 tiles, one per CU, 4 wavefronts each)"}
    return {"workload": "context_kv_proj 4096x7168 . 7168x2880 (bf16 MFMA, fp32 acc)",
            "mfma_ceiling": ceiling,
            "us": round(us, 2), "p90_us": round(p90, 2), "TFLOPs": round(flops / us / 1e6, 1),
            "frac_of_peak": round(flops / us / 1e6 / 2500.0, 4),
            "torch_matmul_us_stream_events": round(statistics.median(ref), 2),
            "with_epilogue_us_stream_events": round(statistics.median(e2e), 2),
            "weight_transpose": {"us": round(tr_us, 2), "p90_us": round(tr_p90, 2),
                                 "bytes": 2 * 7168 * L * W * 2,
                                 "GBps": round(2 * 7168 * L * W * 2 / tr_us / 1e3, 1),
                                 "note": "[7168, 2880] -> [2880, 7168], once per weight"},
            "with_weight_transpose_and_epilogue_us_stream_events": round(statistics.median(e2e_tr),
                                                                         2)}


# ----------------------------------------------------------- CPU baseline --
def cpu_baseline(torch):
    """The oracle (plain serial C) on a bounded sample of one step's work:
    the grouped fp8 insert of 5 layers x 8192 tokens, one gather of 8192
    tokens and the fp8 pack of 6144 tokens x 64 heads (about 10 s serial on
    a current server core)."""
    import numpy as np

    import oracle
    from fp8_paged_insert_amd import synth

    oracle.build(force=False)
    g = synth.gen(5)
    n, npk = 8192, 6144
    kv = synth.bf16_normal((L, n, R), g).view(torch.int16).numpy().view(np.uint16)
    pe = synth.bf16_normal((L, n, P), g).view(torch.int16).numpy().view(np.uint16)
    caches = [np.zeros((256, 64, W), np.uint8) for _ in range(L)]
    sm = np.stack([np.random.default_rng(l).permutation(256 * 64)[:n]
                   for l in range(L)]).astype(np.int64)
    scales = np.linspace(0.5, 2.0, L).astype(np.float32)
    c = synth.context_cache(seed=55, num_blocks=256, num_ctx=8192)
    cache_np, slots_np = c["cache"].numpy(), c["src_slots"].numpy()
    kvb = synth.bf16_normal((npk, 64, 256), g).view(torch.int16).numpy().view(np.uint16)

    t0 = time.perf_counter()
    oracle.insert_grouped(kv, pe, sm, caches, scales)
    t1 = time.perf_counter()
    ws = oracle.gather(cache_np, slots_np, 0.5)
    t2 = time.perf_counter()
    oracle.pack(kvb[..., :128], ws[:npk, 512:], kvb[..., 128:], mode=oracle.PACK_KEY_V_FP8)
    t3 = time.perf_counter()
    nbytes = insert_bytes(L, n) + gather_bytes(8192) + pack_fp8_bytes(npk, 64)
    secs = t3 - t0
    out = {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"insert 5x{n} tokens ({t1 - t0:.2f}s) + gather 8192 tokens "
                     f"({t2 - t1:.2f}s) + fp8 pack {npk} tokens x 64 heads ({t3 - t2:.2f}s); "
                     f"{nbytes} algorithmic bytes in {secs:.2f}s, serial C",
           "host_cpu": _cpu_model()}
    # The same sample on all host cores: disjoint token slices on threads (the
    # oracle's C calls release the GIL; its lazily filled code tables are
    # already filled by the serial run above, so the threads only read them).
    from concurrent.futures import ThreadPoolExecutor

    nt = max(1, min(16, os.cpu_count() or 1))
    cuts = lambda m: [(m * i // nt, m * (i + 1) // nt) for i in range(nt)]
    caches2 = [np.zeros_like(c) for c in caches]
    ins = [(np.ascontiguousarray(kv[:, a:b]), np.ascontiguousarray(pe[:, a:b]),
            np.ascontiguousarray(sm[:, a:b])) for a, b in cuts(n)]
    gat = [np.ascontiguousarray(slots_np[a:b]) for a, b in cuts(8192)]
    pk = [(kvb[a:b, :, :128], ws[a:b, 512:], kvb[a:b, :, 128:]) for a, b in cuts(npk)]
    with ThreadPoolExecutor(max_workers=nt) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda x: oracle.insert_grouped(x[0], x[1], x[2], caches2, scales), ins))
        list(ex.map(lambda x: oracle.gather(cache_np, x, 0.5), gat))
        list(ex.map(lambda x: oracle.pack(x[0], x[1], x[2], mode=oracle.PACK_KEY_V_FP8), pk))
        psecs = time.perf_counter() - t0
    out["all_cores"] = {"value": round(nbytes / psecs / 1e9, 4), "unit": "GB/s", "cores": nt,
                        "sample": f"the same sample split by tokens over {nt} threads, "
                                  f"{psecs:.2f}s"}
    return out


def oracle_components(torch, projection_rows=4096):
    """The oracle (plain serial C, one core) timed beside the components the
    step does not contain, each on a bounded sample of its workload and in the
    component's unit (inputs are generated outside the timed calls)."""
    import numpy as np

    import oracle
    from fp8_paged_insert_amd import synth

    oracle.build(force=False)

    def u16(t):
        return np.ascontiguousarray(t.contiguous().view(torch.int16).numpy().view(np.uint16))

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    out = {}
    # small-batch grouped insert: the whole 5 x 4 workload, 200 calls
    d = synth.small_batch_fp8("cpu")
    caches = [c.numpy().copy() for c in d["caches"]]
    kv, pe = u16(d["kv_c"]), u16(d["k_pe"])
    sm, sc = np.ascontiguousarray(d["slot_mapping"].numpy()), d["scales"].numpy()
    secs = timed(lambda: [oracle.insert_grouped(kv, pe, sm, caches, sc) for _ in range(200)])
    out["small_batch_insert"] = {"value": round(secs / 200 * 1e6, 2), "unit": "us/call",
                                 "cores": 1,
                                 "sample": "the whole 5 x 4 workload, 200 calls through the "
                                           "oracle's Python wrapper"}
    del caches
    # projection: 16 rows of the 4096 x 7168 . 7168 x 2880 product (float64 sums)
    g = synth.gen(3)
    x = u16(synth.bf16_normal((16, 7168), g))
    w = u16(synth.bf16_normal((7168, L * W), g, std=0.02))
    secs = timed(lambda: oracle.gemm_rows(x, w))
    flops = 2 * 16 * 7168 * L * W
    out["context_kv_proj"] = {"value": round(flops / secs / 1e9, 3), "unit": "GFLOP/s",
                              "cores": 1, "sample": f"16 of the 4096 rows ({secs:.2f}s)"}
    # the whole 169 GFLOP product on all host cores (row slices on threads;
    # the oracle's C calls release the GIL): its wall time
    from concurrent.futures import ThreadPoolExecutor

    nt = max(1, min(16, os.cpu_count() or 1))
    rows = projection_rows
    xa = u16(synth.bf16_normal((rows, 7168), g))
    with ThreadPoolExecutor(max_workers=nt) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda i: oracle.gemm_rows(xa, w, np.arange(rows * i // nt,
                                                                 rows * (i + 1) // nt,
                                                                 dtype=np.int64)),
                    range(nt)))
        secs = time.perf_counter() - t0
    what = "the whole 4096-row product" if rows == 4096 else f"{rows} of the 4096 rows"
    out["context_kv_proj"]["all_cores"] = {
        "value": round(2 * rows * 7168 * L * W / secs / 1e9, 3), "unit": "GFLOP/s", "cores": nt,
        "sample": f"{what} in {secs:.2f}s (wall) over {nt} threads"}
    # context epilogue: 5 layers x 1024 tokens
    e = synth.context_epilogue("cpu", num_tokens=1024, num_blocks=16, with_gemm=False)
    caches = [c.numpy().copy() for c in e["caches"]]
    akv, gam = u16(e["all_kv"]), u16(e["gamma"])
    pos, slm = e["positions"].numpy(), np.ascontiguousarray(e["slot_mapping"].numpy())
    secs = timed(lambda: oracle.ctx_kv_epilogue(akv, gam, e["eps"], pos, slm, caches,
                                                e["scales"].numpy()))
    out["context_epilogue"] = {"value": round(epilogue_bytes(L, 1024) / secs / 1e9, 4),
                               "unit": "GB/s", "cores": 1,
                               "sample": f"5 layers x 1024 of the 4096 tokens ({secs:.2f}s)"}
    # chunk merge: 2048 tokens x 64 heads x 128
    m = synth.attention_partials("cpu", num_tokens=2048, heads=64, head_dim=128, chunks=2)
    acc, part = u16(m["outs"][0]), u16(m["outs"][1])
    lacc = np.ascontiguousarray(m["lses"][0].numpy())
    plse = np.ascontiguousarray(m["lses"][1].numpy())
    secs = timed(lambda: oracle.merge_chunk(acc, lacc, part, plse, oracle.MERGE_ACCUMULATE))
    out["chunk_merge"] = {"value": round(merge_bytes(2048, 64) / secs / 1e9, 4), "unit": "GB/s",
                          "cores": 1, "sample": f"2048 of the 16384 tokens ({secs:.2f}s)"}
    # new-token epilogue, fp8 (plain cast): 512 tokens x 64 heads
    n = synth.new_tokens("cpu", num_tokens=512)
    q, kvb, lat = u16(n["q"]), u16(n["kvb"]), u16(n["kv"])
    h = [np.ascontiguousarray(a) for a in (q[..., :128], q[..., 128:], kvb[..., :128],
                                           lat[:, :R], lat[:, R:], kvb[..., 128:])]
    cache, slots = n["cache"].numpy().copy(), n["slots"].numpy()
    valid = int((slots >= 0).sum())
    secs = timed(lambda: oracle.new_token_epilogue(
        h[0], h[1], h[2], h[3], h[4], n["positions"].numpy(), v=h[5], mode=oracle.PACK_KEY_V_FP8,
        cache=cache, slots=slots, cache_scale=float(n["cache_scale"][0])))
    out["new_token_epilogue"] = {"value": round(new_token_bytes(512, 64, True, valid) / secs / 1e9,
                                                4),
                                 "unit": "GB/s", "cores": 1,
                                 "sample": f"fp8, 512 of the 8192 tokens x 64 heads ({secs:.2f}s)"}
    return out


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip() + f" ({os.cpu_count()} logical CPUs visible)"
    except OSError:
        pass
    return None


# ------------------------------------------------------------------- main --
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device-to-device copy 3 times (reference "
                         "kernel of known traffic for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this path has no "
              "multi-GPU leg: each rank would run the same kernels on its own share.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import fp8_paged_insert_amd as mk

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 1 << 30,
                          "copy_calibration_bytes_written": 1 << 30, "launches": 3}))
        return
    mk.lib()
    wl = LongContext(torch, mk, dev)
    for _ in range(args.warmup):
        wl.step()
    wl.arm_timing(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        wl.step(time_pack=True)
    torch.cuda.synchronize()
    secs = time.perf_counter() - t0
    ms_per_step = secs / args.steps * 1e3
    nbytes = wl.bytes_per_step()
    value = nbytes * args.steps / secs / 1e9

    per_window = len(wl.kvb) - 1
    joint_us = statistics.mean(e0.elapsed_time(e1) * 1e3 / per_window for e0, e1 in wl.pack_windows)
    joint_b = pack_fp8_bytes(wl.chunk, wl.heads) + gather_bytes(wl.chunk)
    achieved = joint_b / joint_us / 1e3
    roofline = {"bound": "hbm", "kernel": "pack_gather_kernel",
                "launch": "fp8 full-key + V pack of one 8192-token x 64-head chunk and the "
                          "dequantising gather of the next chunk's 8192 latent rows",
                "achieved": round(achieved, 1),
                "timing": "HIP events recorded on the launch stream before the first and "
                          "after the last of the 15 back-to-back joint launches of every timed "
                          "step; the window / 15 (the gaps between launches included)",
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(), "bytes_per_launch": joint_b,
                "avg_launch_us": round(joint_us, 2),
                "launches": len(wl.pack_windows) * per_window}

    result = {
        "metric": "grouped MLA KV insert/pack: effective HBM GB/s (% of peak); "
                  "µs/launch small batch",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded, generated on the device)",
        "config": {"workload": "long-context stress: grouped fp8 insert 5 layers x 16384 tokens "
                               "into [4096,64,576] caches + 16 chunks x 8192 tokens of fp8 gather "
                               "and fp8 full-key/V pack (64 heads, [8192,64,256] kv_b_proj output)",
                   "io": "bf16 inputs, fp8 e4m3fn caches / keys / V, bf16 gather workspace; "
                         "conversions computed in fp32",
                   "launches": "insert; gather of chunk 0; 15 joint launches (pack of chunk c + "
                               "gather of chunk c + 1); pack of chunk 15",
                   "bytes_per_step": nbytes, "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
    }
    # the same work with the pack as a grid-stride loop over a capped grid (64
    # workgroups of 256 threads per compute unit: 16384 workgroups, 2.5 chunks
    # per thread, against 40960 for one chunk per thread; the fastest of the
    # caps 16, 32 and 64 per compute unit, which the components report), and
    # with the gather and the pack of every chunk as launches of their own
    cap = 64 * torch.cuda.get_device_properties(dev).multi_processor_count
    for name, mb, fn in (("capped_grid_step", cap, lambda: wl.step(max_blocks=cap)),
                         ("separate_launch_step", 0, wl.step_separate)):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        csecs = time.perf_counter() - t0
        result[name] = {
            "max_blocks": mb, "ms_per_step": round(csecs / args.steps * 1e3, 4),
            "GBps": round(nbytes * args.steps / csecs / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes * args.steps / csecs / 1e9 / HBM_PEAK_GBS, 4)}
    del wl
    torch.cuda.empty_cache()
    if not args.no_components:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        result["copy_ceiling"] = copy_ceiling(torch, mk, dev, flush)
        # the dominant kernel against the measured ceiling for its traffic: a
        # streaming kernel with the pack's read:write mix at the pack's size,
        # timed the same way (events recorded by the launch, after a flush)
        mix = result["copy_ceiling"]["stream_mix_2to1_pack_size"]
        result["roofline"]["measured_ceiling"] = {
            "GBps": mix["GBps"], "what": "copy_ceiling.stream_mix_2to1_pack_size",
            "frac": round(roofline["achieved"] / mix["GBps"], 4)}
        comps = {"small_batch_insert": small_batch(torch, mk, dev),
                 "single_layer_insert": single_layer_component(torch, mk, dev),
                 "context_pack": context_pack_component(torch, mk, dev, flush),
                 "context_epilogue": epilogue_component(torch, mk, dev, flush),
                 "cache_dtypes": cache_dtype_component(torch, mk, dev, flush),
                 "chunk_merge": merge_component(torch, mk, dev, flush),
                 "new_token_epilogue": new_token_component(torch, mk, dev, flush),
                 "context_kv_proj": projection_component(torch, mk, dev, flush)}
        result["components"] = comps
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(torch)
        if "components" in result:
            for name, o in oracle_components(torch).items():
                result["components"][name]["cpu_oracle"] = o
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
