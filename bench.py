#!/usr/bin/env python3
"""Benchmark of split-KV MLA decode (partial + merge) on one MI355X.

A step is one mla_decode call (split-KV partial kernel + merge kernel) over one batch of
synthetic, HBM-resident inputs; the host plan is built once, outside the timed region,
and its cost is reported separately. The headline workload is H12 q1 B16 128K
(16 requests x 131072 tokens, 12 heads, one query token), the metric's shape; `value`
is the achieved KV-read bandwidth (KV bytes read once per call / time per call) with
the native one-wave split plan, and the pages' fixed split_kv = 6 plan is reported next
to it. `roofline` covers the dominant kernel (the split-KV partial kernel), timed with
HIP events on the stream it is launched on; `cpu_baseline` is the fp64 oracle on a
bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--all]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from decode_attention_gather_amd import inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "µs per MLA decode call + achieved KV-read HBM GB/s (H12 q1 B16 128K)"
HEADLINE = "m_b16_h12_q1_128k"


def algorithmic_bytes(case) -> dict:
    """Bytes the method must move once: every visible token's 576-byte cache row, the
    query rows, the block-table entries, and the outputs (BF16 O + fp32 LSE)."""
    B = case.batch
    rows = case.rows
    pages = int(sum((int(L) + 31) // 32 for L in case.kv_lens.tolist()))
    kv = case.kv_bytes
    q = rows * 576
    bt = pages * 4
    out = rows * (512 * 2 + 4)
    return dict(kv=kv, q=q, bt=bt, out=out, partial_in=kv + q + bt, total=kv + q + bt + out)


def profiled_traffic(config: str):
    """HBM bytes per partial-kernel launch from the committed rocprofv3 counter summary
    (profiles/partial_kernel_<config>.md), or None when the kernel source changed since
    the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"partial_kernel_{config}.md")
    src = os.path.join(ROOT, "decode_attention_gather_amd", "csrc", "partial.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        k, sep, v = line.strip().partition(": ")
        if sep and k in ("traffic_bytes_per_launch", "kernel_source_sha256"):
            fields[k] = v.strip()
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("kernel_source_sha256") != sha or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def time_calls(fn, steps, warmup, stream, reps=1):
    """`warmup` untimed calls, then `reps` timed runs of exactly `steps` back-to-back calls,
    each bracketed by torch.cuda.synchronize() and one pair of HIP events on `stream`.
    Returns the per-run time per call (us) and the host wall time of the last run."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    per = []
    wall = 0.0
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per.append(a.elapsed_time(b) * 1e3 / steps)
    return np.array(per), wall


def bench_config(mla, name, split_kv, steps, warmup, dc=None, case=None):
    case = case if case is not None else inputs.make_config(name)
    dc = dc if dc is not None else mla.to_device(case)
    t0 = time.perf_counter()
    plan = mla.Plan(dc.kv_lens_host, q_len=case.q_len, num_heads=case.num_heads,
                    split_kv=split_kv, max_split_kv=128)
    plan_us = (time.perf_counter() - t0) * 1e6
    info, splits, chunk = plan.info()
    ws = plan.alloc_workspace()
    rows = case.rows
    o = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        mla.decode(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale,
                   dc.output_scale, ws, o, lse, stream)

    def partial_only():
        mla.partial(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale, ws, stream)

    per_call, wall = time_calls(call, steps, warmup, stream)
    per_partial, _ = time_calls(partial_only, steps, warmup, stream)
    by = algorithmic_bytes(case)
    us = float(np.median(per_call))
    us_p = float(np.median(per_partial))
    return dict(
        config=name, split_kv=split_kv, splits=sorted(set(splits)), work_items=info.work_items,
        merge_groups=info.merge_groups, plan_us=round(plan_us, 1),
        us_per_call=round(us, 2), us_min=round(float(per_call.min()), 2),
        us_max=round(float(per_call.max()), 2),
        kv_gbs=round(by["kv"] / (us * 1e-6) / 1e9, 1),
        partial_us=round(us_p, 2), partial_gbs=round(by["partial_in"] / (us_p * 1e-6) / 1e9, 1),
        merge_us=round(us - us_p, 2), wall_s=round(wall, 4), bytes=by, case=case, dc=dc)


def cpu_baseline(case, budget_rows=None):
    """The fp64 oracle on a bounded sample of the workload's rows (all host cores)."""
    import oracle
    threads = oracle.hw_threads()
    nrows = min(budget_rows or case.rows, case.rows)
    rows = inputs.sample_rows(case, nrows)
    t0 = time.perf_counter()
    oracle.mla_decode(case.q, case.kv, case.block_table, case.kv_lens, q_len=case.q_len,
                      num_heads=case.num_heads, softmax_scale=float(np.float32(case.softmax_scale)),
                      output_scale=case.output_scale, rows=rows, nthreads=threads)
    dt = time.perf_counter() - t0
    call_s = dt * case.rows / len(rows)
    return dict(value=round(case.kv_bytes / call_s / 1e9, 4), unit="GB/s", cores=threads,
                kind="oracle", us_per_call=round(call_s * 1e6, 1),
                sample=f"{len(rows)} of {case.rows} rows (every KV token of each), "
                       f"{dt:.2f} s on {threads} threads, scaled to the full call")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=HEADLINE, choices=sorted(inputs.CONFIGS))
    ap.add_argument("--all", action="store_true", help="also time every workload (stderr)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for HBM counter scaling)")
    ap.add_argument("--planner-only", action="store_true", help="skip the fixed-split plan")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the decode path has no multi-GPU sharding in this "
              "build (requests, heads and KV splits would shard across GPUs; see DESIGN.md). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        x = torch.ones(1 << 28, dtype=torch.int32, device="cuda")  # 1 GiB
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": x.numel() * 4, "copies": 3}))
        return
    from decode_attention_gather_amd import mla

    name = args.config
    print(f"[bench] generating {name}", file=sys.stderr, flush=True)
    case = inputs.make_config(name)
    dc = mla.to_device(case)
    native = bench_config(mla, name, 0, args.steps, args.warmup, dc=dc, case=case)
    print(f"[bench] planner plan: {native['us_per_call']} us/call", file=sys.stderr, flush=True)
    fixed = None
    if case.split_kv and not args.planner_only:
        fixed = bench_config(mla, name, case.split_kv, args.steps, args.warmup, dc=dc, case=case)
        print(f"[bench] split_kv={case.split_kv}: {fixed['us_per_call']} us/call", file=sys.stderr,
              flush=True)
    cpu = None if args.no_cpu else cpu_baseline(case)

    by = native["bytes"]
    achieved = by["partial_in"] / (native["partial_us"] * 1e-6) / 1e9
    res = {
        "metric": METRIC,
        "value": native["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(native["us_per_call"] / 1e3, 5),
        "us_per_call": native["us_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 in (fp32 accumulate), bf16 out",
        "data": "synthetic: N(0,1) cast to E4M3, seeded random block table",
        "config": {"workload": name, "batch": case.batch, "kv_len": int(case.kv_lens.max()),
                   "heads": case.num_heads, "q_len": case.q_len, "page": 32,
                   "split_plan": "planner (one wave, cap 128)", "splits": native["splits"],
                   "work_items": native["work_items"], "parallelism": "1 GPU"},
        "plan_us": native["plan_us"],
        "merge_us": native["merge_us"],
        "fixed_split": None if fixed is None else {
            "split_kv": fixed["split_kv"], "us_per_call": fixed["us_per_call"],
            "kv_gbs": fixed["kv_gbs"], "partial_us": fixed["partial_us"],
            "work_items": fixed["work_items"]},
        "roofline": {"bound": "hbm", "kernel": "partial_kernel",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(name),
                     "bytes_per_launch": by["partial_in"], "us_per_launch": native["partial_us"]},
        "cpu_baseline": None if cpu is None else {k: cpu[k] for k in
                                                  ("value", "unit", "cores", "kind", "sample",
                                                   "us_per_call")},
    }
    if args.all:
        for other in sorted(inputs.CONFIGS):
            if other == name:
                continue
            c = inputs.make_config(other)
            for sk in ([0, c.split_kv] if c.split_kv else [0]):
                r = bench_config(mla, other, sk, args.steps, args.warmup, case=c)
                print("[bench-all] " + json.dumps({k: v for k, v in r.items()
                                                   if k not in ("case", "dc", "bytes")}),
                      file=sys.stderr, flush=True)
                del r
            torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
