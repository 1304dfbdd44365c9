#!/usr/bin/env python3
"""Benchmark of the paged-attention decode step on one MI355X.

A step is one pass of the decode hot path over one synthetic batch already
resident in HBM: ``pa_reshape_and_cache`` writes each sequence's new K/V token
into its cache slot, then ``pa_decode`` (partition kernel + partition merge
kernel) attends every query head over its paged context.  The default workload is the
Qwen3-0.6B-shaped decode batch (128 sequences, 16 query / 8 KV heads, head_dim
128, 16-token blocks shuffled over a 300k-block pool, context lengths uniform
in [200, 2048], bf16).

Prints one JSON line.  ``value`` is effective KV GB/s: the logical K+V bytes
the batch attends over (every context token of every sequence, once) divided
by the step time.  The ``roofline`` object reports the decode kernels alone,
timed with HIP events on the stream they run on; ``cpu_baseline`` times the
CPU oracle on the host cores.
"""
from __future__ import annotations

import argparse
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
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["paged_kv_cache_324_amd/csrc/decode_impl.h",
                  "paged_kv_cache_324_amd/csrc/pa_device.h"]


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, partition: int):
    """HBM bytes per decode launch from the committed counter summary, if it is current."""
    path = os.path.join(PROFILES, f"decode_{workload}_p{partition}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != kernel_source_sha():
        return None
    return float(val.group(1))


def cpu_baseline(b, budget_s: float = 10.0):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    kc, vc = b.k_blocks.copy(), b.v_blocks.copy()
    reps, kv, seqs = 0, 0, 0
    wall0, cpu0 = time.perf_counter(), time.process_time()
    # One pass over the whole batch, then more passes while the budget lasts.
    while True:
        oracle.reshape_and_cache(b.key_new, b.value_new, kc, vc, b.slot_mapping_compact)
        oracle.paged_decode(b.q, kc, vc, b.block_tables_compact, b.context_lens, b.scale, b.dtype)
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
            "host_cpus_visible": len(os.sched_getaffinity(0))}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3_0p6b_decode")
    ap.add_argument("--partition", type=int, default=None, help="tokens per context partition")
    ap.add_argument("--unfused", action="store_true",
                    help="step = pa_reshape_and_cache + pa_decode (two launches) instead of the "
                         "fused pa_decode_step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--copy-kernel-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (--steps "
                         "times): the reference kernel for scaling HBM byte counters")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the decode path shards by sequence or KV head with no exchange, see DESIGN.md",
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
    partition = cfg["partition"] if args.partition is None else args.partition

    t_gen = time.perf_counter()
    b = make_config(args.workload)
    print(f"[bench] generated {args.workload} in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr,
          flush=True)
    dt = torch.bfloat16 if b.dtype == "bf16" else torch.float16
    dev = torch.device("cuda:0")
    shape = (b.NB, b.BS, b.Hkv, b.D)
    k_cache = torch.full(shape, -1, dtype=torch.int16, device=dev)
    v_cache = torch.full(shape, -1, dtype=torch.int16, device=dev)
    idx = torch.from_numpy(b.phys_ids).to(dev)
    k_cache[idx] = torch.from_numpy(b.k_blocks.view(np.int16)).to(dev)
    v_cache[idx] = torch.from_numpy(b.v_blocks.view(np.int16)).to(dev)
    k_cache, v_cache = k_cache.view(dt), v_cache.view(dt)

    def dev16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(dt)

    q, key_new, value_new = dev16(b.q), dev16(b.key_new), dev16(b.value_new)
    slot = torch.from_numpy(b.slot_mapping).to(dev)
    tables = torch.from_numpy(b.block_tables).to(dev)
    lens = torch.from_numpy(b.context_lens).to(dev)
    out = torch.empty_like(q)
    workspace = pa.decode_workspace(b.B, b.Hq, b.D, b.max_context_len, partition, dev)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    # Longest-first visiting order of the sequences, computed on the host from
    # the lengths the caller knows (the library's pa_decode_order).
    order = torch.from_numpy(pa.pa_decode_order(b.context_lens)).to(dev)

    def step():
        if args.unfused:
            pa.pa_reshape_and_cache(key_new, value_new, k_cache, v_cache, slot, stream=stream)
            pa.pa_decode(out, q, k_cache, v_cache, tables, lens, b.scale, b.max_context_len,
                         partition, workspace=workspace, seq_order=order, stream=stream)
        else:
            pa.pa_decode_step(out, q, key_new, value_new, slot, k_cache, v_cache, tables, lens,
                              b.scale, b.max_context_len, partition, workspace=workspace,
                              seq_order=order, stream=stream)

    def decode_only():
        step() if not args.unfused else pa.pa_decode(
            out, q, k_cache, v_cache, tables, lens, b.scale, b.max_context_len, partition,
            workspace=workspace, seq_order=order, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps back to back, nothing else on the stream.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Kernel timing for the roofline: each pa_decode call (partition kernel +
    # merge kernel) bracketed by HIP events recorded on the stream it runs on.
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    for i in range(args.steps):
        events[i][0].record(stream)
        decode_only()
        events[i][1].record(stream)
    torch.cuda.synchronize()
    decode_ms = np.array([s.elapsed_time(e) for s, e in events])

    ms_per_step = wall / args.steps * 1e3
    kv = b.kv_bytes()
    value = kv / (ms_per_step * 1e-3) / 1e9
    dec_avg_s = float(decode_ms.mean()) * 1e-3
    achieved = kv / dec_avg_s / 1e9
    traffic = recorded_traffic(args.workload, partition)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "num_seqs": b.B, "num_heads": b.Hq,
                   "num_kv_heads": b.Hkv, "head_dim": b.D, "block_size": b.BS,
                   "pool_blocks": b.NB, "context_lens": "uniform[%d,%d]" % tuple(cfg["lens"]),
                   "seed": cfg["seed"], "partition_size": partition,
                   "kv_bytes_per_step": kv},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "seqs_per_s": round(b.B / (ms_per_step * 1e-3), 1),
        "decode_us": {"mean": round(float(decode_ms.mean()) * 1e3, 2),
                      "p10": round(float(np.percentile(decode_ms, 10)) * 1e3, 2),
                      "p50": round(float(np.median(decode_ms)) * 1e3, 2),
                      "p90": round(float(np.percentile(decode_ms, 90)) * 1e3, 2)},
        "roofline": {"bound": "hbm", "kernel": "pa_decode (partition + merge kernels)",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(b, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
