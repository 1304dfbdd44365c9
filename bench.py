#!/usr/bin/env python3
"""Benchmark of the paged-attention decode step on one MI355X.

A step is one pass of the decode hot path over one synthetic batch already
resident in HBM: each sequence's new K/V token is stored into its cache slot and
every query head attends over its paged context (``pa_decode_step``, one
launch; with ``--unfused``, ``pa_reshape_and_cache`` then ``pa_decode``).  The
default workload is the Qwen3-0.6B-shaped decode batch (128 sequences, 16 query
/ 8 KV heads, head_dim 128, 16-token blocks shuffled over a 300k-block pool,
context lengths uniform in [200, 2048], bf16).

Protocol: ``--warmup`` untimed steps, then exactly ``--steps`` timed steps, each
preceded by a flush read of ``--flush-mb`` MiB (so no K/V byte comes from the
Infinity Cache or an L2) and bracketed by HIP events on the stream it runs on.
``value`` is effective KV GB/s over the median step: the logical K+V bytes the
batch attends over (every context token of every sequence, once) divided by the
step time; ``roofline.achieved`` is the same bytes over the mean of the same
durations.  Warm back-to-back steps, a streaming-read ceiling and (for split
contexts) the partition and merge kernels timed on their own are reported as
labelled extras; ``cpu_baseline`` times the CPU oracle on the host cores, and
``parity`` compares the step's output with the oracle's.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn decode effective KV GB/s (% of HBM peak) + sequences/s, 1 GPU"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16/fp16 matrix-core peak
PROFILES = os.path.join(ROOT, "profiles")
# Sources of the decode kernels; a counter summary holds their hash and counts
# only while they are unchanged.
KERNEL_SOURCES = ["paged_kv_cache_324_amd/csrc/decode_impl.h",
                  "paged_kv_cache_324_amd/csrc/decode_mfma_impl.h",
                  "paged_kv_cache_324_amd/csrc/mfma.h",
                  "paged_kv_cache_324_amd/csrc/pa_device.h"]
# Sources of the INT8 decode kernel (its merge is the 16-bit one).
KERNEL_SOURCES_INT8 = ["paged_kv_cache_324_amd/csrc/decode_int8.hip",
                       "paged_kv_cache_324_amd/csrc/decode_impl.h",
                       "paged_kv_cache_324_amd/csrc/mfma.h",
                       "paged_kv_cache_324_amd/csrc/pa_device.h"]
# Sources of the chunked-prefill kernel and of the fused rotary + cache-write kernel.
KERNEL_SOURCES_PREFILL = ["paged_kv_cache_324_amd/csrc/prefill.hip",
                          "paged_kv_cache_324_amd/csrc/prefill_impl.h",
                          "paged_kv_cache_324_amd/csrc/mfma.h",
                          "paged_kv_cache_324_amd/csrc/pa_device.h"]
KERNEL_SOURCES_ROPE = ["paged_kv_cache_324_amd/csrc/rope_reshape.hip",
                       "paged_kv_cache_324_amd/csrc/pa_device.h"]


def kernel_source_sha(sources=None) -> str:
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from(summary: str, sources):
    """HBM bytes per launch recorded in profiles/<summary>, while the hash of `sources`
    still matches the one recorded with it (else None: the kernel changed since)."""
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != kernel_source_sha(sources):
        return None
    return float(val.group(1))


def recorded_traffic(workload: str, partition: int, int8: bool = False):
    """HBM bytes per decode launch from the committed counter summary, if it is current."""
    tag = "_int8" if int8 else ""
    return traffic_from(f"decode_{workload}{tag}_p{partition}_counters.md",
                        KERNEL_SOURCES_INT8 if int8 else KERNEL_SOURCES)


def cpu_baseline(b, budget_s: float = 10.0, gpu_out_bits=None):
    """The oracle, as it stands, on a bounded sample of the same workload.  With the GPU
    step's output given, the first pass's oracle output also yields the headline parity."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    kc, vc = b.k_blocks.copy(), b.v_blocks.copy()
    reps, kv, seqs = 0, 0, 0
    parity = None
    wall0, cpu0 = time.perf_counter(), time.process_time()
    # One pass over the whole batch, then more passes while the budget lasts.
    while True:
        oracle.reshape_and_cache(b.key_new, b.value_new, kc, vc, b.slot_mapping_compact)
        ref = oracle.paged_decode(b.q, kc, vc, b.block_tables_compact, b.context_lens, b.scale,
                                  b.dtype)
        if parity is None and gpu_out_bits is not None:
            t_par = time.perf_counter()
            parity = parity_stats(gpu_out_bits, ref, b.dtype)
            wall0 += time.perf_counter() - t_par          # not part of the oracle's time
        reps += 1
        kv += b.kv_bytes()
        seqs += b.B
        if time.perf_counter() - wall0 >= budget_s:
            break
    wall = time.perf_counter() - wall0
    cpu = time.process_time() - cpu0
    return {"value": round(kv / wall / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{reps} full pass(es) of the {b.B}-sequence batch (reshape_and_cache + "
                      f"float64 decode), {wall:.1f} s wall, {cpu:.1f} s CPU",
            "seqs_per_s": round(seqs / wall, 2),
            "host_cpus_visible": len(os.sched_getaffinity(0))}, parity


def _stats_us(ms):
    ms = np.asarray(ms, dtype=np.float64)
    return {"n": int(ms.size), "mean": round(float(np.mean(ms)) * 1e3, 2),
            "p10": round(float(np.percentile(ms, 10)) * 1e3, 2),
            "p50": round(float(np.median(ms)) * 1e3, 2),
            "p90": round(float(np.percentile(ms, 90)) * 1e3, 2)}


def parity_stats(got_bits, ref, dtype):
    """Headline parity, computed in the CPU-baseline leg from the oracle output it has just
    produced: max-abs and relative L2 of the GPU output against the float64 oracle, the
    count of |o_ref| >= 4, and the largest error in excess of rounding o_ref to 16 bits."""
    import oracle
    from workloads import to_u16
    got = oracle.decode_u16(got_bits, dtype)
    err = np.abs(got - ref)
    rounded = oracle.decode_u16(to_u16(ref.astype(np.float32), dtype), dtype)
    return {"what": "headline step output vs the float64 oracle, every element",
            "max_abs": float(err.max()), "rel_l2": float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
            "n_ref_abs_ge_4": int((np.abs(ref) >= 4).sum()),
            "max_excess_over_16bit_rounding": float((err - np.abs(rounded - ref)).max()),
            "bar": {"max_abs": 1.5e-2, "rel_l2": 5e-3}}


def prefill_flops(b) -> float:
    """Algorithmic FLOPs of a chunk: 2 D per visible key for QK^T and 2 D for PV, every query head."""
    n = b.n_new.astype(np.int64)
    c = b.context_lens.astype(np.int64) - n
    visible = (n * c + n * (n + 1) // 2).sum()
    return float(4 * b.D * b.Hq * visible)


def upload(torch, b, dev):
    """Device pool of b.NB blocks, NaN everywhere except the referenced blocks."""
    import types
    dt = torch.bfloat16 if b.dtype == "bf16" else torch.float16
    shape = (b.NB, b.BS, b.Hkv, b.D)
    k_cache = torch.full(shape, -1, dtype=torch.int16, device=dev)
    v_cache = torch.full(shape, -1, dtype=torch.int16, device=dev)
    idx = torch.from_numpy(b.phys_ids).to(dev)
    k_cache[idx] = torch.from_numpy(b.k_blocks.view(np.int16)).to(dev)
    v_cache[idx] = torch.from_numpy(b.v_blocks.view(np.int16)).to(dev)

    def dev16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(dt)

    return types.SimpleNamespace(
        k_cache=k_cache.view(dt), v_cache=v_cache.view(dt), q=dev16(b.q), key_new=dev16(b.key_new),
        value_new=dev16(b.value_new), slot=torch.from_numpy(b.slot_mapping).to(dev),
        tables=torch.from_numpy(b.block_tables).to(dev),
        lens=torch.from_numpy(b.context_lens).to(dev),
        qsl=torch.from_numpy(b.query_start_loc).to(dev))


class Timer:
    """The timing protocol.  A timed call is preceded by a flush: the library's read of a
    buffer of `flush_mb` MiB (default 1 GiB, four times the 256 MB Infinity Cache), so no
    operand is served from the MALL or an L2, and, being a read, it leaves no dirty line
    to be written back during the call.  The call's duration is the interval between two
    HIP events on its stream that the library's kernels record from their own dispatch
    end timestamps (pa_set_kernel_events): the end of the flush and the end of the call's
    last kernel.  No other packet sits between them, so the interval is the call's
    device time plus the dispatch gap to its first kernel, the gap a stream of calls
    also has."""

    def __init__(self, torch, pa, dev, flush_mb: int):
        self.torch = torch
        self.pa = pa
        self.stream = torch.cuda.current_stream(dev)
        self.flush_bytes = max(1, int(flush_mb)) << 20
        self.flush_buf = torch.zeros(self.flush_bytes, dtype=torch.uint8, device=dev)

    def flush(self):
        self.pa.pa_cache_flush(self.flush_buf, stream=self.stream)

    def _events(self, n):
        torch = self.torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in ev:              # a torch event holds no HIP event before its first record
            e.record(self.stream)
        torch.cuda.synchronize()
        return ev

    def cold(self, fn, n):
        """Device times (ms) of n calls, each after a flush: flush end to call end."""
        marks, ends = self._events(n), self._events(n)
        try:
            for a, b in zip(marks, ends):
                self.pa.pa_set_kernel_events(None, a)
                self.flush()
                self.pa.pa_set_kernel_events(None, b)
                fn()
        finally:
            self.pa.pa_set_kernel_events()
        self.torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in zip(marks, ends)])

    def warm(self, fn, n):
        """Device times (ms) of n calls issued back to back: the end of each call to the end
        of the next (n + 1 calls)."""
        ends = self._events(n + 1)
        try:
            for b in ends:
                self.pa.pa_set_kernel_events(None, b)
                fn()
        finally:
            self.pa.pa_set_kernel_events()
        self.torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in zip(ends[:-1], ends[1:])])

    def back_to_back(self, fn, n):
        """Wall time per call (ms) of n calls issued back to back, nothing else on the stream."""
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n * 1e3

    def warmup(self, fn, calls: int, min_ms: float = 0.0):
        """At least `calls` calls, and more until at least `min_ms` of them have run."""
        torch = self.torch
        t0 = time.perf_counter()
        done = 0
        while done < calls or (time.perf_counter() - t0) * 1e3 < min_ms:
            for _ in range(max(1, calls if done < calls else 16)):
                fn()
                done += 1
            torch.cuda.synchronize()

    def stream_read_ceiling(self):
        """Streaming read rates of this device, as references (never a denominator):
        non-temporal loads over 4 GiB (pa_stream_read), the HBM read rate a kernel that
        streams its operands once can reach; and the flush itself (plain loads, which
        allocate cache lines) timed back to back over its buffer."""
        big = self.torch.empty(4 << 30, dtype=self.torch.uint8, device=self.flush_buf.device)

        def read():
            self.pa.pa_stream_read(big, stream=self.stream)

        for _ in range(3):
            read()
        ms_nt = float(np.median(self.warm(read, 10)))
        del big
        for _ in range(3):
            self.flush()
        ms = float(np.median(self.warm(self.flush, 10)))
        return {"kernel": "pa_stream_read over 4096 MiB (non-temporal loads)",
                "GBps": round((4 << 30) / (ms_nt * 1e-3) / 1e9, 1),
                "us_p50": round(ms_nt * 1e3, 2),
                "flush_read": {"kernel": f"pa_cache_flush over {self.flush_bytes >> 20} MiB "
                                         "(plain loads)",
                               "GBps": round(self.flush_bytes / (ms * 1e-3) / 1e9, 1),
                               "us_p50": round(ms * 1e3, 2)}}


# Secondary workloads run a fixed number of cold steps after a time-based warm-up,
# independent of --steps, so a short driver run reports them as a long one does.
SECONDARY_STEPS = 50
SECONDARY_WARMUP_MS = 100.0


def resolve_partition(pa, cfg, b):
    """The workload's split-K partition, or the library's choice for this device."""
    if cfg["partition"] is not None:
        return cfg["partition"]
    return pa.pa_decode_partition_hint(b.B, b.Hkv, b.max_context_len, b.BS)


def run_decode(pa, torch, b, partition, steps, warmup, unfused, dev, timer, warmup_ms=0.0):
    """Decode steps on the batch: `warmup` untimed steps, then exactly `steps` cold steps
    (the timed region), then the labelled extras: warm back-to-back steps and, for a split
    decode, its two phases (pa_decode_partitions cold, pa_decode_merge over the partials
    it left) timed on their own."""
    d = upload(torch, b, dev)
    out = torch.empty_like(d.q)
    workspace = pa.decode_workspace(b.B, b.Hq, b.D, b.max_context_len, partition, dev)
    stream = timer.stream
    # Longest-first visiting order of the sequences, computed on the host from
    # the lengths the caller knows (the library's pa_decode_order).
    order = torch.from_numpy(pa.pa_decode_order(b.context_lens)).to(dev)

    def decode():
        pa.pa_decode(out, d.q, d.k_cache, d.v_cache, d.tables, d.lens, b.scale, b.max_context_len,
                     partition, workspace=workspace, seq_order=order, stream=stream)

    def step():
        if unfused:
            pa.pa_reshape_and_cache(d.key_new, d.value_new, d.k_cache, d.v_cache, d.slot,
                                    stream=stream)
            decode()
        else:
            pa.pa_decode_step(out, d.q, d.key_new, d.value_new, d.slot, d.k_cache, d.v_cache,
                              d.tables, d.lens, b.scale, b.max_context_len, partition,
                              workspace=workspace, seq_order=order, stream=stream)

    timer.warmup(step, warmup, warmup_ms)
    step_ms = timer.cold(step, steps)                     # the timed region
    out_bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    warm_ms = timer.back_to_back(step, steps)
    warm_dev_ms = timer.warm(step, steps)
    split = bool(partition) and b.max_context_len > partition
    phases = None
    if split:
        def partitions():
            pa.pa_decode_partitions(out, d.q, d.k_cache, d.v_cache, d.tables, d.lens, b.scale,
                                    b.max_context_len, partition, workspace=workspace,
                                    seq_order=order, stream=stream)

        def merge():
            pa.pa_decode_merge(out, d.lens, b.max_context_len, partition, workspace,
                               seq_order=order, stream=stream)

        k2 = timer.cold(partitions, steps)
        partitions()
        phases = {"k2_partitions_us": _stats_us(k2),
                  "k3_merge_us": _stats_us(timer.warm(merge, steps)),
                  "note": "k2: pa_decode_partitions alone, cold (no new-token store); k3: "
                          "pa_decode_merge alone over the partials k2 left, back to back "
                          "(the partials resident, as after k2 in a step)"}
    # The library runs the matrix-core kernel for 2+ query heads per KV head at
    # head_dim 128, the vector kernel otherwise.
    kern = "decode_mfma_kernel" if (b.G >= 2 and b.D == 128) else "decode_partition_kernel"
    name = ("pa_decode" if unfused else "pa_decode_step") + (
        f" ({kern} + merge kernel)" if split else f" (one {kern} launch)")
    return {"step_ms": step_ms, "warm_ms": warm_ms, "warm_dev_ms": warm_dev_ms,
            "kernel_name": name, "phases": phases, "out_bits": out_bits}


def int8_kv_bytes(b) -> int:
    """Bytes of the quantised K and V one decode reads: a code per element and one fp32
    scale per (token, KV head), for keys and values."""
    return int(b.context_lens.astype(np.int64).sum()) * b.Hkv * (b.D + 4) * 2


def run_decode_int8(pa, torch, b, partition, steps, dev, timer):
    """Decode over an INT8 cache: each step quantises the new tokens into their slots and
    attends, in one launch (pa_decode_step_int8); the same step as two launches
    (pa_reshape_and_cache_int8, pa_decode_int8) is timed beside it.  The cache is filled
    with the batch's cached tokens, quantised by the library, before timing."""
    dt = torch.bfloat16 if b.dtype == "bf16" else torch.float16

    def dev16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(dt)

    kc = torch.zeros((b.NB, b.Hkv, b.BS, b.D), dtype=torch.int8, device=dev)   # head-major
    vc = torch.zeros_like(kc)
    ks = torch.zeros((b.NB, b.Hkv, b.BS), dtype=torch.float32, device=dev)
    vs = torch.zeros_like(ks)
    comp = []
    for i in range(b.B):                      # cached positions, each physical slot once
        t = np.arange(int(b.context_lens[i]) - int(b.n_new[i]))
        comp.append(b.block_tables_compact[i, t // b.BS].astype(np.int64) * b.BS + t % b.BS)
    comp = np.unique(np.concatenate(comp))
    for lo in range(0, comp.size, 1 << 18):
        c = comp[lo:lo + (1 << 18)]
        phys = b.phys_ids[c // b.BS].astype(np.int64) * b.BS + c % b.BS
        pa.pa_reshape_and_cache_int8(dev16(b.k_blocks.reshape(-1, b.Hkv, b.D)[c]),
                                     dev16(b.v_blocks.reshape(-1, b.Hkv, b.D)[c]), kc, vc, ks, vs,
                                     torch.from_numpy(phys).to(dev))
    q, knew, vnew = dev16(b.q), dev16(b.key_new), dev16(b.value_new)
    slot = torch.from_numpy(b.slot_mapping).to(dev)
    tables = torch.from_numpy(b.block_tables).to(dev)
    lens = torch.from_numpy(b.context_lens).to(dev)
    out = torch.empty_like(q)
    workspace = pa.decode_workspace(b.B, b.Hq, b.D, b.max_context_len, partition, dev)
    stream = timer.stream
    order = torch.from_numpy(pa.pa_decode_order(b.context_lens)).to(dev)
    torch.cuda.synchronize(dev)

    def decode():
        pa.pa_decode_int8(out, q, kc, vc, ks, vs, tables, lens, b.scale, b.max_context_len,
                          partition, workspace=workspace, seq_order=order, stream=stream)

    def two_launches():
        pa.pa_reshape_and_cache_int8(knew, vnew, kc, vc, ks, vs, slot, stream=stream)
        decode()

    def step():        # the new tokens quantised into their slots and attended, one launch
        pa.pa_decode_step_int8(out, q, knew, vnew, slot, kc, vc, ks, vs, tables, lens, b.scale,
                               b.max_context_len, partition, workspace=workspace,
                               seq_order=order, stream=stream)

    timer.warmup(step, 5, SECONDARY_WARMUP_MS)
    step_ms = timer.cold(step, steps)
    timer.warmup(two_launches, 5, SECONDARY_WARMUP_MS)
    two_ms = timer.cold(two_launches, steps)
    split = bool(partition) and b.max_context_len > partition
    merge_ms = None
    if split:
        step()
        merge_ms = timer.warm(lambda: pa.pa_decode_merge(out, lens, b.max_context_len, partition,
                                                         workspace, seq_order=order,
                                                         stream=stream), steps)
    name = "pa_decode_step_int8 (decode_int8_kernel" + (
        " + merge kernel)" if split else ", one launch)")
    return {"step_ms": step_ms, "two_launch_ms": two_ms, "kernel_name": name, "merge_ms": merge_ms}


def contiguous_shard(b, nshards, s):
    """Shard s of a context split into nshards contiguous runs of whole blocks: its
    physical block tables [B][W] (-1 padded) and its per-sequence token counts."""
    nb = -(-b.context_lens.astype(np.int64) // b.BS)
    per = -(-nb // nshards)
    lo, hi = np.minimum(s * per, nb), np.minimum((s + 1) * per, nb)
    W = max(1, int((hi - lo).max()))
    tables = np.full((b.B, W), -1, np.int32)
    lens = np.zeros(b.B, np.int32)
    for i in range(b.B):
        tables[i, :hi[i] - lo[i]] = b.block_tables[i, lo[i]:hi[i]]
        if hi[i] > lo[i]:
            lens[i] = min(int(b.context_lens[i]), int(hi[i]) * b.BS) - int(lo[i]) * b.BS
    return tables, lens


def run_decode_cp(pa, torch, b, nshards, steps, dev, timer):
    """Context-parallel decode as one device of an nshards-way group sees it: the partial
    decode of its shard (the first, which holds the most tokens) at its real shape, then
    the merge of all nshards partial rows.  All shards' partials are computed once
    before timing so the merge reads real rows; the exchange between devices is not
    part of a one-device step."""
    d = upload(torch, b, dev)
    pa.pa_reshape_and_cache(d.key_new, d.value_new, d.k_cache, d.v_cache, d.slot)
    o = torch.empty((nshards,) + tuple(d.q.shape), dtype=d.q.dtype, device=dev)
    ml = torch.empty((nshards, b.B, b.Hq, 2), dtype=torch.float32, device=dev)
    shards = []
    for s in range(nshards):
        tables, lens = contiguous_shard(b, nshards, s)
        mx = max(int(lens.max()), 1)
        part = pa.pa_decode_partition_hint(b.B, b.Hkv, mx, b.BS)
        ws = pa.decode_workspace(b.B, b.Hq, b.D, mx, part, dev)
        shards.append((torch.from_numpy(tables).to(dev), torch.from_numpy(lens).to(dev), mx, part,
                       ws, torch.from_numpy(pa.pa_decode_order(lens)).to(dev), lens))
        pa.pa_decode_partial(o[s], ml[s], d.q, d.k_cache, d.v_cache, shards[-1][0], shards[-1][1],
                             b.scale, mx, part, workspace=ws, seq_order=shards[-1][5])
    tables, lens_d, mx, part, ws, order, lens = shards[0]
    out = torch.empty_like(d.q)
    stream = timer.stream
    torch.cuda.synchronize(dev)

    def partial():
        pa.pa_decode_partial(o[0], ml[0], d.q, d.k_cache, d.v_cache, tables, lens_d, b.scale, mx,
                             part, workspace=ws, seq_order=order, stream=stream)

    def merge():
        pa.pa_merge_partials(out, o, ml, stream=stream)

    def step():
        partial()
        merge()

    timer.warmup(step, 5, SECONDARY_WARMUP_MS)
    step_ms = timer.cold(step, steps)
    shard_bytes = int(lens.astype(np.int64).sum()) * b.Hkv * b.D * 2 * 2
    merge_bytes = b.B * b.Hq * (nshards * (b.D * 2 + 8) + b.D * 2)
    return {"step_ms": step_ms, "partial_ms": timer.cold(partial, steps),
            "merge_ms": timer.warm(merge, steps), "partition_size": part,
            "shard_kv_bytes": shard_bytes, "merge_bytes": merge_bytes,
            "shard_tokens": [int(lens.min()), int(lens.max())]}


def rope_bytes(b) -> int:
    """Algorithmic bytes of the fused rotary step over the workload's new tokens: queries
    read and written, keys and values read and written to the cache, and one cos and one
    sin row (float32, head_dim / 2) per token."""
    T = len(b.slot_mapping)
    return T * (b.Hq * b.D * 2 * 2 + b.Hkv * b.D * 2 * 4 + b.D // 2 * 4 * 2)


def run_rope(pa, torch, b, steps, dev, timer):
    """pa_rope_reshape_and_cache over the workload's new tokens at their positions (queries
    rotated in place), beside the plain pa_reshape_and_cache of the same tokens."""
    from workloads import rope_tables
    d = upload(torch, b, dev)
    T = len(b.slot_mapping)
    pos = np.concatenate([np.arange(int(L) - int(n), int(L))
                          for L, n in zip(b.context_lens, b.n_new)]).astype(np.int64)
    cos, sin = rope_tables(int(pos.max()) + 1, b.D)
    cos_d, sin_d = torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev)
    pos_d = torch.from_numpy(pos).to(dev)
    q = d.q if d.q.shape[0] == T else torch.zeros((T, b.Hq, b.D), dtype=d.q.dtype, device=dev)
    stream = timer.stream

    def fused():
        pa.pa_rope_reshape_and_cache(q, d.key_new, d.value_new, d.k_cache, d.v_cache, pos_d, cos_d,
                                     sin_d, d.slot, stream=stream)

    def plain():
        pa.pa_reshape_and_cache(d.key_new, d.value_new, d.k_cache, d.v_cache, d.slot, stream=stream)

    timer.warmup(fused, 5, SECONDARY_WARMUP_MS)
    fused_ms = timer.cold(fused, steps)
    timer.warmup(plain, 5, SECONDARY_WARMUP_MS)
    return {"step_ms": fused_ms, "plain_ms": timer.cold(plain, steps), "tokens": T}


def run_graph(pa, torch, b, steps, warmup, dev, timer):
    """A serving-style decode step: the rotary embedding of q and of the new key, the cache
    write of the new key and value, and decode.  Timed as two launches
    (pa_rope_reshape_and_cache, then pa_decode) and as the one fused launch
    (pa_decode_step_rope), each eager and as replays of the step captured in a HIP graph."""
    from workloads import rope_tables
    d = upload(torch, b, dev)
    pos = torch.from_numpy(b.context_lens.astype(np.int64) - 1).to(dev)
    cos, sin = rope_tables(int(b.max_context_len) + 1, b.D)
    cos_d, sin_d = torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev)
    out = torch.empty_like(d.q)
    partition = pa.pa_decode_partition_hint(b.B, b.Hkv, b.max_context_len, b.BS)
    ws = pa.decode_workspace(b.B, b.Hq, b.D, b.max_context_len, partition, dev)
    order = torch.from_numpy(pa.pa_decode_order(b.context_lens)).to(dev)

    def step():
        pa.pa_rope_reshape_and_cache(d.q, d.key_new, d.value_new, d.k_cache, d.v_cache, pos, cos_d,
                                     sin_d, d.slot)
        pa.pa_decode(out, d.q, d.k_cache, d.v_cache, d.tables, d.lens, b.scale, b.max_context_len,
                     partition, workspace=ws, seq_order=order)

    def fused():
        pa.pa_decode_step_rope(out, d.q, d.key_new, d.value_new, d.slot, pos, cos_d, sin_d,
                               d.k_cache, d.v_cache, d.tables, d.lens, b.scale, b.max_context_len,
                               partition, workspace=ws, seq_order=order)

    def eager_and_graph(fn):
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for _ in range(warmup):
                fn()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize(dev)
        eager_ms = timer.back_to_back(fn, steps)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(warmup):
            g.replay()
        return eager_ms, timer.back_to_back(g.replay, steps)

    eager_ms, graph_ms = eager_and_graph(step)
    fused_ms, fused_graph_ms = eager_and_graph(fused)
    return {"eager_ms": eager_ms, "graph_ms": graph_ms, "fused_ms": fused_ms,
            "fused_graph_ms": fused_graph_ms, "partition_size": partition}


def run_prefill(pa, torch, b, steps, dev, timer):
    d = upload(torch, b, dev)
    out = torch.empty_like(d.q)
    stream = timer.stream
    order = torch.from_numpy(pa.pa_decode_order(b.context_lens)).to(dev)

    def reshape():
        pa.pa_reshape_and_cache(d.key_new, d.value_new, d.k_cache, d.v_cache, d.slot, stream=stream)

    def prefill():
        pa.pa_prefill_chunk(out, d.q, d.k_cache, d.v_cache, d.tables, d.lens, d.qsl,
                            b.max_query_len, b.scale, seq_order=order, stream=stream)

    def step():
        reshape()
        prefill()

    timer.warmup(step, 5, SECONDARY_WARMUP_MS)
    step_ms = timer.cold(step, steps)
    return {"step_ms": step_ms, "prefill_ms": timer.cold(prefill, steps),
            "reshape_ms": timer.cold(reshape, steps)}


def _p50(ms) -> float:
    return float(np.median(ms))


def _hbm_roofline(kernel, nbytes, ms, traffic):
    """Algorithmic bytes over the mean duration of the same timed calls."""
    achieved = nbytes / (float(np.mean(ms)) * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic}


def secondary_entry(pa, torch, entry, dev, timer):
    """One entry of the secondary report, measured by the same cold protocol with a fixed
    number of steps and a time-based warm-up."""
    from workloads import CONFIGS, make_config
    name, _, variant = entry.partition(":")
    c2 = CONFIGS[name]
    t_gen = time.perf_counter()
    b2 = make_config(name)
    print(f"[bench] generated {name} in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr,
          flush=True)
    n = SECONDARY_STEPS
    if variant.startswith("cp"):
        ns = int(variant[2:])
        r2 = run_decode_cp(pa, torch, b2, ns, n, dev, timer)
        kb = r2["shard_kv_bytes"]
        kern = "decode_mfma_kernel" if (b2.G >= 2 and b2.D == 128) else "decode_partition_kernel"
        return {
            "step": f"pa_decode_partial (shard 0 of {ns}) + pa_merge_partials ({ns} shards)",
            "partition_size": r2["partition_size"], "steps": n,
            "ms_per_step": round(_p50(r2["step_ms"]), 5), "step_us": _stats_us(r2["step_ms"]),
            "shard_tokens": r2["shard_tokens"], "shard_kv_bytes": kb,
            "merge_bytes": r2["merge_bytes"], "partial_us": _stats_us(r2["partial_ms"]),
            "merge_us": _stats_us(r2["merge_ms"]),
            "merge_GBps": round(r2["merge_bytes"] / (float(np.mean(r2["merge_ms"])) * 1e-3) / 1e9, 2),
            "roofline": _hbm_roofline(f"pa_decode_partial ({kern})", kb, r2["partial_ms"],
                                      traffic_from(f"decode_{name}_cp{ns}_p{r2['partition_size']}"
                                                   "_counters.md", KERNEL_SOURCES))}
    if variant == "graph":
        r2 = run_graph(pa, torch, b2, n, 10, dev, timer)
        kv2 = b2.kv_bytes()
        return {
            "step": "rotary embedding + cache write + decode: two launches "
                    "(pa_rope_reshape_and_cache, pa_decode) vs one (pa_decode_step_rope), "
                    "each eager and as HIP-graph replays, warm back to back",
            "partition_size": r2["partition_size"], "steps": n,
            "eager_us_per_step": round(r2["eager_ms"] * 1e3, 2),
            "graph_us_per_step": round(r2["graph_ms"] * 1e3, 2),
            "graph_speedup": round(r2["eager_ms"] / r2["graph_ms"], 3),
            "fused_eager_us_per_step": round(r2["fused_ms"] * 1e3, 2),
            "fused_graph_us_per_step": round(r2["fused_graph_ms"] * 1e3, 2),
            "fused_speedup": round(r2["eager_ms"] / r2["fused_ms"], 3),
            "fused_effective_GBps": round(kv2 / (r2["fused_ms"] * 1e-3) / 1e9, 2)}
    if variant == "rope":
        r2 = run_rope(pa, torch, b2, n, dev, timer)
        rb = rope_bytes(b2)
        plain_bytes = 2 * 2 * r2["tokens"] * b2.Hkv * b2.D * 2
        return {
            "step": "pa_rope_reshape_and_cache (queries rotated in place, keys rotated into "
                    "the cache, values copied)", "tokens": r2["tokens"], "steps": n,
            "ms_per_step": round(_p50(r2["step_ms"]), 5), "algorithmic_bytes": rb,
            "rope_us": _stats_us(r2["step_ms"]),
            "plain_reshape_and_cache_us": _stats_us(r2["plain_ms"]),
            "plain_reshape_and_cache_GBps": round(plain_bytes / (_p50(r2["plain_ms"]) * 1e-3) / 1e9, 1),
            "roofline": _hbm_roofline("rope_reshape_kernel", rb, r2["step_ms"],
                                      traffic_from(f"rope_reshape_{name}_counters.md",
                                                   KERNEL_SOURCES_ROPE))}
    if variant == "int8":
        p2 = resolve_partition(pa, c2, b2)
        r2 = run_decode_int8(pa, torch, b2, p2, n, dev, timer)
        kb = int8_kv_bytes(b2)
        t = _p50(r2["step_ms"]) * 1e-3
        e = {"step": "pa_decode_step_int8 (quantising store + decode, one launch)",
             "partition_size": p2, "steps": n, "ms_per_step": round(t * 1e3, 5),
             "step_us": _stats_us(r2["step_ms"]),
             "two_launch_us": _stats_us(r2["two_launch_ms"]),
             "int8_kv_bytes": kb, "effective_GBps": round(kb / t / 1e9, 2),
             "note": "effective_GBps counts the INT8 codes and scales read; the same step over a "
                     "16-bit cache would read kv_bytes_16bit",
             "kv_bytes_16bit": b2.kv_bytes(),
             "seqs_per_s": round(b2.B / t, 1),
             "roofline": _hbm_roofline(r2["kernel_name"], kb, r2["step_ms"],
                                       recorded_traffic(name, p2, int8=True))}
        if r2["merge_ms"] is not None:
            e["k3_merge_us"] = _stats_us(r2["merge_ms"])
        return e
    if c2["kind"] == "prefill":
        r2 = run_prefill(pa, torch, b2, n, dev, timer)
        flops = prefill_flops(b2)
        tfl = flops / (float(np.mean(r2["prefill_ms"])) * 1e-3) / 1e12
        return {
            "step": "pa_reshape_and_cache (all new tokens) + pa_prefill_chunk", "steps": n,
            "ms_per_step": round(_p50(r2["step_ms"]), 5), "step_us": _stats_us(r2["step_ms"]),
            "prefill_us": _stats_us(r2["prefill_ms"]),
            "reshape_and_cache_us": _stats_us(r2["reshape_ms"]),
            "reshape_and_cache_GBps": round(
                2 * 2 * len(b2.slot_mapping) * b2.Hkv * b2.D * 2 / (_p50(r2["reshape_ms"]) * 1e-3)
                / 1e9, 1),
            "algorithmic_gflop": round(flops / 1e9, 2),
            "roofline": {"bound": "mfma", "kernel": "prefill_kernel", "achieved": round(tfl, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic_from(f"prefill_{name}_counters.md",
                                                 KERNEL_SOURCES_PREFILL)}}
    p2 = resolve_partition(pa, c2, b2)
    r2 = run_decode(pa, torch, b2, p2, n, 5, False, dev, timer, warmup_ms=SECONDARY_WARMUP_MS)
    kv2 = b2.kv_bytes()
    t = _p50(r2["step_ms"]) * 1e-3
    e = {"step": "pa_decode_step", "partition_size": p2, "steps": n, "ms_per_step": round(t * 1e3, 5),
         "step_us": _stats_us(r2["step_ms"]), "effective_GBps": round(kv2 / t / 1e9, 2),
         "unique_kv_bytes": b2.unique_kv_bytes(), "kv_bytes": kv2,
         "warm_back_to_back_us": round(r2["warm_ms"] * 1e3, 2),
         "roofline": _hbm_roofline(r2["kernel_name"], kv2, r2["step_ms"],
                                   recorded_traffic(name, p2))}
    if r2["phases"]:
        e["phases"] = r2["phases"]
    return e


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3_0p6b_decode")
    ap.add_argument("--seed", type=int, default=None,
                    help="seed of the headline workload's inputs (default: the workload's own)")
    ap.add_argument("--flush-mb", type=int, default=1024,
                    help="MiB read before every timed call to evict the Infinity Cache and L2s")
    ap.add_argument("--partition", type=int, default=None, help="tokens per context partition")
    ap.add_argument("--unfused", action="store_true",
                    help="step = pa_reshape_and_cache + pa_decode (two launches) instead of the "
                         "fused pa_decode_step")
    ap.add_argument("--secondary",
                    default="llama2_70b_decode_bs16,llama2_70b_decode_bs32,long_splitk_decode,"
                            "chunked_prefill,qwen3_0p6b_decode:int8,llama2_70b_decode_bs16:int8,"
                            "long_splitk_decode:int8,long_splitk_decode:cp8,chunked_prefill:rope,"
                            "qwen3_0p6b_decode:rope,tiny_decode:graph,qwen3_0p6b_decode:graph",
                    help="comma-separated extra workloads reported beside the headline; "
                         "a ':int8' suffix runs the workload over an INT8 KV cache, ':cpN' "
                         "as one device of an N-way context-parallel group, ':rope' times the "
                         "fused rotary embedding + cache write of its new tokens, ':graph' a "
                         "rotary + decode step as two launches and as one fused launch, each eager "
                         "and as HIP-graph replays")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--copy-kernel-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (--steps "
                         "times): the reference kernel for scaling HBM byte counters")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); decode shards "
              "by sequence or KV head with no exchange, so N GPUs run N independent batches",
              file=sys.stderr)
        return 2

    import torch
    import paged_kv_cache_324_amd as pa
    from workloads import CONFIGS, make_config

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.copy_kernel_bytes:
        src = torch.ones(args.copy_kernel_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt_s = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"copy_bytes": args.copy_kernel_bytes, "steps": args.steps,
                          "us_per_copy": round(dt_s * 1e6, 2),
                          "read_plus_write_GBps": round(2 * args.copy_kernel_bytes / dt_s / 1e9, 1)}))
        return 0
    pa.load_library()
    cfg = CONFIGS[args.workload]
    if cfg["kind"] != "decode":
        print("bench.py: the headline workload is a decode batch", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    timer = Timer(torch, pa, dev, args.flush_mb)

    t_gen = time.perf_counter()
    seed = cfg["seed"] if args.seed is None else args.seed
    b = make_config(args.workload, seed=seed)
    print(f"[bench] generated {args.workload} in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr,
          flush=True)
    partition = resolve_partition(pa, cfg, b) if args.partition is None else args.partition
    r = run_decode(pa, torch, b, partition, args.steps, args.warmup, args.unfused, dev, timer)
    print("[bench] headline timed", file=sys.stderr, flush=True)
    kv = b.kv_bytes()
    t = _p50(r["step_ms"]) * 1e-3
    value = kv / t / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "num_seqs": b.B, "num_heads": b.Hq,
                   "num_kv_heads": b.Hkv, "head_dim": b.D, "block_size": b.BS,
                   "pool_blocks": b.NB, "context_lens": "uniform[%d,%d]" % tuple(cfg["lens"]),
                   "seed": seed, "partition_size": partition,
                   "step": "pa_reshape_and_cache + pa_decode" if args.unfused else
                           "pa_decode_step (new-token store + decode, one launch)",
                   "seq_order": "longest context first (pa_decode_order on the host)",
                   "kv_bytes_per_step": kv},
        "protocol": (f"{args.warmup} warm-up steps, then {args.steps} timed steps, each after a "
                     f"{args.flush_mb} MiB flush read (pa_cache_flush); a step's time runs from "
                     "the flush kernel's end to the step's last kernel's end, both HIP events on "
                     "the stream recorded from the kernels' dispatch timestamps "
                     "(pa_set_kernel_events); value and ms_per_step from the median, "
                     "roofline.achieved from the mean of the same durations"),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "seqs_per_s": round(b.B / t, 1),
        "step_us": _stats_us(r["step_ms"]),
        "warm_back_to_back": {"us_per_step": round(r["warm_ms"] * 1e3, 2),
                              "GBps": round(kv / (r["warm_ms"] * 1e-3) / 1e9, 2),
                              "device_us": _stats_us(r["warm_dev_ms"]),
                              "note": "labelled extra: the same step issued back to back "
                                      "without flushes; us_per_step is wall time per step, "
                                      "device_us the interval between consecutive steps' ends"},
        "kernels": r["phases"] or {"k2": r["kernel_name"], "k3": "none (no context split)"},
        "stream_read_ceiling": timer.stream_read_ceiling(),
        "roofline": _hbm_roofline(r["kernel_name"], kv, r["step_ms"],
                                  recorded_traffic(args.workload, partition)),
    }
    secondary = {}
    for entry in [x for x in args.secondary.split(",") if x]:
        # Hand the previous workload's pools (up to ~20 GB) back to the device, so that
        # each entry's caches are fresh allocations rather than pieces of cached segments.
        torch.cuda.synchronize(dev)
        gc.collect()
        torch.cuda.empty_cache()
        secondary[entry] = secondary_entry(pa, torch, entry, dev, timer)
    if secondary:
        result["secondary"] = secondary
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"], result["parity"] = cpu_baseline(b, args.cpu_budget, r["out_bits"])
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
