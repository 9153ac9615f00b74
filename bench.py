#!/usr/bin/env python3
"""Benchmark of split-KV MLA decode (partial + merge) on one MI355X.

A step is one mla_decode call (split-KV partial kernel + merge kernel) over one batch of
synthetic, HBM-resident inputs; host plans are built once, outside the timed region,
and their cost is reported separately. The headline workload is H12 q1 B16 128K
(16 requests x 131072 tokens, 12 heads, one query token). `value` is the achieved
KV-read bandwidth (KV bytes read once per call / time per call) with the native
one-wave split plan, timed first; the pages' fixed split_kv = 6 plan is reported beside
it, and the q = 8 sibling of the workload (same KV, 8 causal query tokens) as `q8`.
Before anything is timed, about a second of the headline's calls brings the clocks up;
every timed loop then follows ~0.2 s of its own untimed calls, since the clocks drop
within tens of milliseconds of idle or lighter load (a plan with fewer work items).

`roofline` covers the dominant kernel (the split-KV partial kernel), timed with HIP
events on the stream it is launched on; `cpu_baseline` is the fp64 oracle on a bounded
sample of the same workload. Per-call times come from one event between consecutive
calls (median, p10, p90); `ms_per_step` is the whole timed region divided by the steps.

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
FP8_MFMA_PEAK_TFLOPS = 5000.0   # dense FP8 MFMA peak of the MI355X
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense BF16 MFMA peak of the MI355X


def mfma_peak(kv_dtype: str) -> float:
    return BF16_MFMA_PEAK_TFLOPS if kv_dtype == "bf16" else FP8_MFMA_PEAK_TFLOPS


def dominant_kernel(kv_dtype: str, rows: int):
    """(kernel name, source file) of the partial kernel a plan launches."""
    if kv_dtype == "bf16":
        if rows > 32:
            return "partial_bf16_wide_kernel", "partial_bf16_wide.hip"
        return "partial_bf16_kernel", "partial_bf16.hip"
    if rows > 32:
        return "partial_wide_kernel", "partial_wide.hip"
    return "partial_kernel", "partial.hip"
FLOP_PER_ROW_TOKEN = 2 * (576 + 512)  # QK^T over 576 dims + PV over 512 dims
METRIC = "µs per MLA decode call + achieved KV-read HBM GB/s (H12 q1 B16 128K)"
HEADLINE = "m_b16_h12_q1_128k"
COLD_BYTES = 512 << 20          # written between calls to evict the 256 MB MALL


def algorithmic_bytes(case) -> dict:
    """Bytes the method must move once: every visible token's cache row (576 bytes in
    E4M3, 1152 in BF16), the query rows, the block-table entries, and the outputs (BF16
    O + fp32 LSE)."""
    rows = case.rows
    pages = int(sum((int(L) + 31) // 32 for L in case.kv_lens.tolist()))
    kv = case.kv_bytes
    q = rows * 576 * case.elem_bytes
    bt = pages * 4
    out = rows * (512 * 2 + 4)
    return dict(kv=kv, q=q, bt=bt, out=out, partial_in=kv + q + bt, total=kv + q + bt + out)


def algorithmic_flops(kv_lens, q_len, num_heads) -> int:
    """2176 flop per (row, visible token); query j of q sees L - q + j + 1 tokens."""
    tok = sum(int(L) - q_len + j + 1 for L in kv_lens for j in range(q_len))
    return tok * num_heads * FLOP_PER_ROW_TOKEN


def profiled_traffic(config: str, kernel: str = "partial_kernel", source: str = "partial.hip"):
    """HBM bytes per partial-kernel launch from the committed rocprofv3 counter summary
    (profiles/<kernel>_<config>.md), or None when the kernel source changed since the
    counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{config}.md")
    src = os.path.join(ROOT, "decode_attention_gather_amd", "csrc", source)
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


def roofline(name: str, case, by: dict, partial_us: float) -> dict:
    """The `roofline` object for the partial kernel of a workload: MFMA-bound when its
    algorithmic flops per algorithmic byte exceed the ridge (dense MFMA peak / 8 TB/s),
    else HBM-bound; achieved = algorithmic flops or bytes per launch / launch time."""
    kname, ksrc = dominant_kernel(case.kv_dtype, case.q_len * case.num_heads)
    flops = algorithmic_flops(case.kv_lens.tolist(), case.q_len, case.num_heads)
    peak_tf = mfma_peak(case.kv_dtype)  # TFLOP/s
    if flops / by["partial_in"] > peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9):
        achieved = flops / (partial_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "kernel": kname, "achieved": round(achieved, 2),
                "peak": peak_tf, "unit": "TFLOP/s", "frac": round(achieved / peak_tf, 4),
                "flops_per_launch": flops}
    else:
        achieved = by["partial_in"] / (partial_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof.update({"traffic": profiled_traffic(name, kname, ksrc),
                 "bytes_per_launch": by["partial_in"], "us_per_launch": partial_us})
    return roof


def time_steps(fn, steps, warmup, stream):
    """`warmup` untimed calls, then exactly `steps` back-to-back calls bracketed by
    torch.cuda.synchronize(), timed by one HIP event pair on `stream` (nothing else is
    enqueued between the calls). Then a second loop of the same calls with an event
    after every call gives the per-call distribution. Returns (µs per call of the first
    loop, per-call µs array of the second, host wall s of the first)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = a.elapsed_time(b) * 1e3 / steps
    n = min(steps, 50)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(stream)
    for i in range(n):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n)])
    return us, per, wall


def clock_warmup(fn, seconds: float = 1.0) -> int:
    """Untimed calls for about `seconds` of GPU time, so that the clocks have left their
    idle state before the first timed region whatever --warmup is (the first ~100 launches
    after the host has been busy generating inputs run up to 1.5x slow). Returns the
    number of calls."""
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            fn()
        torch.cuda.synchronize()
        n += 50
    return n


def time_cold(fn, calls, stream):
    """Per-call µs with the MALL (and L2) evicted before each call: a 512 MB buffer is
    written between calls, outside the event pair."""
    scratch = torch.empty(COLD_BYTES, dtype=torch.uint8, device="cuda")
    fn()
    torch.cuda.synchronize()
    pairs = []
    for _ in range(calls):
        scratch.fill_(1)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    del scratch
    return np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])


def stats(per):
    return dict(median=round(float(np.median(per)), 2), p10=round(float(np.percentile(per, 10)), 2),
                p90=round(float(np.percentile(per, 90)), 2))


def bench_plan(mla, dc, q, rows, kv_bytes, kv_lens, split_kv, steps, warmup, cold_calls=0):
    """Times mla_decode calls and partial-only launches of one plan."""
    t0 = time.perf_counter()
    plan = mla.Plan(kv_lens, q_len=q.shape[1], num_heads=q.shape[2], split_kv=split_kv,
                    max_split_kv=256, kv_dtype=dc.kv_dtype)
    plan_us = (time.perf_counter() - t0) * 1e6
    info, splits, _ = plan.info()
    ws = plan.alloc_workspace()
    o = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        mla.decode(plan, q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale,
                   dc.output_scale, ws, o, lse, stream)

    def partial_only():
        mla.partial(plan, q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale, ws, stream)

    # each timed loop follows ~0.2 s of its own untimed calls: the clocks drop within tens
    # of ms of lighter load (a plan with fewer work items) or idle, and take ~100 ms of
    # full load to come back
    clock_warmup(call, 0.2)
    us, per, wall = time_steps(call, steps, warmup, stream)
    clock_warmup(partial_only, 0.2)
    us_p, per_p, _ = time_steps(partial_only, steps, warmup, stream)
    res = dict(split_kv=split_kv, splits=sorted(set(splits)), work_items=info.work_items,
               row_tiles=info.row_tiles, merge_groups=info.merge_groups,
               plan_us=round(plan_us, 1), us_per_call=round(us, 2), call=stats(per),
               kv_gbs=round(kv_bytes / (us * 1e-6) / 1e9, 1),
               partial_us=round(us_p, 2), partial=stats(per_p),
               partial_kv_gbs=round(kv_bytes / (us_p * 1e-6) / 1e9, 1),
               merge_us=round(us - us_p, 2), wall_s=round(wall, 4))
    if cold_calls:
        res["cold_mall"] = stats(time_cold(call, cold_calls, stream))
    plan.close()
    return res


def graph_path(mla, dc, q, rows, kv_bytes, steps, warmup):
    """Times the graph-capturable call (device planner + partial + merge, device lengths
    and scales) with the plan's length bound at the batch's longest request."""
    lens = dc.kv_lens_host
    plan = mla.Plan.graph(len(lens), q_len=q.shape[1], num_heads=q.shape[2],
                          max_kv_len=max(lens), kv_dtype=dc.kv_dtype)
    ws = plan.alloc_workspace()
    o = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
    ss = torch.tensor([dc.softmax_scale], dtype=torch.float32, device="cuda")
    os_ = torch.tensor([dc.output_scale], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        mla.decode_graph(plan, q, dc.kv, dc.block_table, dc.kv_lens, ss, os_, ws, o, lse, stream)

    clock_warmup(call, 0.2)
    us, per, _ = time_steps(call, steps, warmup, stream)
    replayed = graph_replay(mla, plan, q, dc, ss, os_, ws, o, lse, kv_bytes)
    info = plan.info()[0]
    plan.close()
    return dict(us_per_call=round(us, 2), call=stats(per), work_item_capacity=info.work_items,
                kv_gbs=round(kv_bytes / (us * 1e-6) / 1e9, 1), replayed=replayed)


def graph_replay(mla, plan, q, dc, ss, os_, ws, o, lse, kv_bytes, calls=20, reps=5):
    """The graph-path call as it is meant to run: `calls` of them captured in one HIP
    graph and replayed (median over `reps` replays), checked against the eager output."""
    torch.cuda.synchronize()
    o_eager, lse_eager = o.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(calls):
                mla.decode_graph(plan, q, dc.kv, dc.block_table, dc.kv_lens, ss, os_, ws, o, lse, s)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) * 1e3 / calls)
    us = float(np.median(per))
    same = bool(torch.equal(o, o_eager) and torch.equal(lse, lse_eager))
    return dict(calls_per_graph=calls, us_per_call=round(us, 2),
                kv_gbs=round(kv_bytes / (us * 1e-6) / 1e9, 1), matches_eager=same)


def q8_sibling(case, q_len=8, seed=20263):
    """Queries for the q = 8 sibling of a workload: N(0, 1) E4M3 rows drawn from their
    own seeded generator, used with the workload's KV cache and block table."""
    g = torch.Generator().manual_seed(seed)
    return inputs.to_e4m3_codes(torch.randn(case.batch, q_len, case.num_heads, 576, generator=g))


def graph_timing(mla, dc, case, calls=100, reps=5):
    """Launch-bound check: `calls` mla_decode calls captured in one HIP graph, replayed,
    against a graph of 2 * `calls` one-element kernels (the launch floor)."""
    plan = mla.Plan(dc.kv_lens_host, q_len=case.q_len, num_heads=case.num_heads, split_kv=0,
                    kv_dtype=dc.kv_dtype)
    ws = plan.alloc_workspace()
    o = torch.empty((case.rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((case.rows,), dtype=torch.float32, device="cuda")
    mla.decode(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale,
               dc.output_scale, ws, o, lse)
    torch.cuda.synchronize()
    o_eager = o.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(calls):
                mla.decode(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale,
                           dc.output_scale, ws, o, lse, s)
    x = torch.zeros(1, device="cuda")
    gf = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(gf, stream=s):
            for _ in range(2 * calls):
                x.add_(1.0)
    torch.cuda.synchronize()

    def replay(gr):
        gr.replay()
        torch.cuda.synchronize()
        best = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            gr.replay()
            b.record()
            torch.cuda.synchronize()
            best.append(a.elapsed_time(b) * 1e3 / calls)
        return float(np.median(best))

    us = replay(g)
    same = bool(torch.equal(o, o_eager))
    floor = replay(gf)
    plan.close()
    return dict(calls_per_graph=calls, us_per_call=round(us, 2),
                floor_us_per_2_kernels=round(floor, 2), graph_matches_eager=same)


def cpu_baseline(case, budget_rows=None, threads=None):
    """The fp64 oracle on a bounded sample of the workload's rows (all host cores, or
    `threads` of them)."""
    import oracle
    threads = threads or oracle.hw_threads()
    nrows = min(budget_rows or case.rows, case.rows)
    rows = inputs.sample_rows(case, nrows)
    t0 = time.perf_counter()
    oracle.mla_decode(case.q, case.kv, case.block_table, case.kv_lens, q_len=case.q_len,
                      num_heads=case.num_heads, softmax_scale=float(np.float32(case.softmax_scale)),
                      output_scale=case.output_scale, rows=rows, nthreads=threads,
                      kv_dtype=case.kv_dtype)
    dt = time.perf_counter() - t0
    # scale by visible row-tokens (the oracle's work), not rows: lengths may differ
    per_req = case.q_len * case.num_heads
    lens = case.kv_lens.tolist()

    def vis(r):
        L = int(lens[r // per_req])
        return L - case.q_len + (r % per_req) // case.num_heads + 1

    total = sum(vis(r) for r in range(case.rows))
    call_s = dt * total / max(sum(vis(r) for r in rows), 1)
    return dict(value=round(case.kv_bytes / call_s / 1e9, 4), unit="GB/s", cores=threads,
                kind="oracle", us_per_call=round(call_s * 1e6, 1),
                sample=f"{len(rows)} of {case.rows} rows (every KV token of each), "
                       f"{dt:.2f} s on {threads} threads, scaled to the full call by "
                       "visible row-tokens")


# row-tokens of fp64 oracle work per workload in `--all` (about 2 s on 16 host threads)
ORACLE_ROW_TOKENS = 50_000_000


def oracle_rows(case, row_tokens: int = ORACLE_ROW_TOKENS) -> int:
    """Rows of a bounded oracle sample: about `row_tokens` row-tokens, at least 16."""
    return min(case.rows, max(16, row_tokens // int(max(case.kv_lens.max(), 1))))


def bench_other(mla, name, steps, warmup, cpu=False):
    """Every plan of one more workload (stderr report and the JSON's `all` list); with
    `cpu`, the oracle on a bounded sample of its rows is attached to the last plan."""
    c = inputs.make_config(name)
    dc = mla.to_device(c)
    by = algorithmic_bytes(c)
    flops = algorithmic_flops(dc.kv_lens_host, c.q_len, c.num_heads)
    out = []
    for sk in ([c.split_kv, 0] if c.split_kv else [0]):
        r = bench_plan(mla, dc, dc.q, c.rows, by["kv"], dc.kv_lens_host, sk, steps, warmup,
                       cold_calls=10)
        r["config"] = name
        r["mfma_util"] = round(flops / (r["us_per_call"] * 1e-6) / 1e12 / mfma_peak(c.kv_dtype), 4)
        out.append(r)
    if name.startswith("c1_"):
        out[-1]["graph"] = graph_timing(mla, dc, c)
    if name.startswith("s_"):
        out[-1]["graph_path"] = graph_path(mla, dc, dc.q, c.rows, by["kv"], steps, warmup)
    if cpu:
        out[-1]["cpu_baseline"] = cpu_baseline(c, oracle_rows(c))
        # one host thread: the whole call for the small workload, else a smaller sample
        out[-1]["cpu_baseline_1thread"] = cpu_baseline(
            c, oracle_rows(c, ORACLE_ROW_TOKENS // 16), threads=1)
    del dc
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", default=HEADLINE, choices=sorted(inputs.CONFIGS))
    ap.add_argument("--all", action="store_true", help="also time every other workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-q8", action="store_true", help="skip the q = 8 sibling")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for HBM counter scaling)")
    ap.add_argument("--planner-only", action="store_true", help="skip the fixed-split plan")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-path timing")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the decode path is not sharded across GPUs "
              "(requests, heads and KV splits are the axes it would shard along, with one "
              "exchange of the per-split partials before the merge). Run with --gpus 1.",
              file=sys.stderr)
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
    by = algorithmic_bytes(case)
    steps, warmup = args.steps, args.warmup

    # clocks up before anything is timed: about a second of the headline's own calls
    wplan = mla.Plan(dc.kv_lens_host, q_len=case.q_len, num_heads=case.num_heads, split_kv=0,
                     max_split_kv=256, kv_dtype=dc.kv_dtype)
    wws = wplan.alloc_workspace()
    wo = torch.empty((case.rows, 512), dtype=torch.bfloat16, device="cuda")
    n_warm = clock_warmup(lambda: mla.decode(wplan, dc.q, dc.kv, dc.block_table, dc.kv_lens,
                                             dc.softmax_scale, dc.output_scale, wws, wo))
    print(f"[bench] clock warm-up: {n_warm} untimed calls", file=sys.stderr, flush=True)
    del wplan, wws, wo

    native = bench_plan(mla, dc, dc.q, case.rows, by["kv"], dc.kv_lens_host, 0, steps, warmup,
                        cold_calls=20)
    print(f"[bench] planner plan: {native['us_per_call']} us/call", file=sys.stderr, flush=True)
    fixed = None
    if case.split_kv and not args.planner_only:
        fixed = bench_plan(mla, dc, dc.q, case.rows, by["kv"], dc.kv_lens_host, case.split_kv,
                           steps, warmup)
        print(f"[bench] split_kv={case.split_kv}: {fixed['us_per_call']} us/call",
              file=sys.stderr, flush=True)
    gpath = None
    if not args.no_graph:
        gpath = graph_path(mla, dc, dc.q, case.rows, by["kv"], steps, warmup)
        print(f"[bench] graph path: {gpath['us_per_call']} us/call", file=sys.stderr, flush=True)

    q8 = None
    if not args.no_q8 and name == HEADLINE:
        q8d = q8_sibling(case).to("cuda")
        rows8 = q8d.shape[0] * q8d.shape[1] * q8d.shape[2]
        flops8 = algorithmic_flops(dc.kv_lens_host, 8, case.num_heads)
        q8 = {"workload": "H12 q8 B16 128K (the headline's KV, 8 causal query tokens)"}
        for key, sk in (("fixed_split", case.split_kv), ("planner", 0)):
            r = bench_plan(mla, dc, q8d, rows8, by["kv"], dc.kv_lens_host, sk, steps, warmup)
            r["mfma_util"] = round(flops8 / (r["us_per_call"] * 1e-6) / 1e12
                                   / FP8_MFMA_PEAK_TFLOPS, 4)
            q8[key] = r
            print(f"[bench] q8 {key}: {r['us_per_call']} us/call", file=sys.stderr, flush=True)
        del q8d

    others = []
    if args.all:
        for other in sorted(inputs.CONFIGS):
            if other == name:
                continue
            for r in bench_other(mla, other, steps, warmup, cpu=not args.no_cpu):
                print("[bench-all] " + json.dumps(r), file=sys.stderr, flush=True)
                others.append(r)

    cpu = None if args.no_cpu else cpu_baseline(case)

    roof = roofline(name, case, by, native["partial_us"])
    res = {
        "metric": METRIC,
        "value": native["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "clock_warmup_calls": n_warm,
        "ms_per_step": round(native["us_per_call"] / 1e3, 5),
        "us_per_call": native["us_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{case.kv_dtype} in (fp32 accumulate), bf16 out",
        "data": ("synthetic: N(0,1) cast to "
                 f"{'BF16' if case.kv_dtype == 'bf16' else 'E4M3'}, seeded random block table"),
        "config": {"workload": name, "batch": case.batch, "kv_len": int(case.kv_lens.max()),
                   "heads": case.num_heads, "q_len": case.q_len, "page": 32,
                   "split_plan": "planner (one XCD-aware wave, cap 256)", "splits": native["splits"],
                   "work_items": native["work_items"], "parallelism": "1 GPU"},
        "call": native["call"],
        "cold_mall": native.get("cold_mall"),
        "plan_us": native["plan_us"],
        "merge_us": native["merge_us"],
        "fixed_split": None if fixed is None else {
            k: fixed[k] for k in ("split_kv", "us_per_call", "call", "kv_gbs", "partial_us",
                                  "work_items")},
        "graph_path": gpath,
        "q8": q8,
        "roofline": roof,
        "cpu_baseline": None if cpu is None else {k: cpu[k] for k in
                                                  ("value", "unit", "cores", "kind", "sample",
                                                   "us_per_call")},
    }
    if others:
        res["all"] = others
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
