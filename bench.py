#!/usr/bin/env python
"""Benchmark of one paged GQA decode step on one MI355X.

A step is paged_attn_decode + paged_attn_merge for a whole batch of one layer
on seeded synthetic inputs already resident in HBM. The default workload is
the long-context batch the target is stated for: B=8 sequences of 131072
tokens, D=256, Hq=24, Hkv=4, 16-token blocks, Q4_0 K and V, blocks shuffled
through one pool (the lucebox PR #555 page's uniform-batch benchmark at its
128K column). Other workloads: --workload NAME (see WORKLOADS).

To keep the 256 MB MALL from serving a step out of cache, the timed loop
rotates over enough independent pool copies that each copy is at least 4x
the MALL between two uses.

Prints ONE JSON line: metric/value (achieved algorithmic HBM GB/s of the
whole step), ms_per_step, a roofline object for the decode kernel (achieved
GB/s against 8 TB/s from hipEvents on the launch stream) and a cpu_baseline
object (the fp64 oracle timed on a bounded sample on the host cores).

  python bench.py [--steps K] [--warmup W] [--settle-ms S] [--workload NAME]
      (defaults 200, 20 and 200: after idle the GPU's clocks take some tens
      of milliseconds of sustained load to settle, so steps first run back to
      back for S ms - recorded in the line as "settle" - then W warmup steps,
      then the K timed steps with no event inside, then the same K steps
      again with events around each decode launch for the kernel split)
  python bench.py --summarize-stats DIR --label NAME   (rocprofv3 --stats CSV -> profiles/)
  python bench.py --summarize-pmc DIR --label NAME     (rocprofv3 --pmc CSVs -> profiles/)
  python bench.py --metadata     (paging-metadata update and copy-on-write timings)
  python bench.py --chunk NAME   (multi-token query attention, see CHUNKS)
  python bench.py --sweep        (one line per batch size 1, 2, 4, 8 of the
                                  uniform Q8_0 4K and Q4_0 32K / 128K workloads)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0          # MI355X HBM3E, public figure
MALL_BYTES = 256 << 20
METRIC = "paged decode step µs + achieved HBM GB/s (% of peak), D=256 Hq=24 Hkv=4"

# name -> (synth workload, B, L, description)
WORKLOADS = {
    "uniform_q4_0_128k_b8": ("uniform_q4_0", 8, 131072, "uniform Q4_0 B=8 L=131072"),
    "uniform_q4_0_32k_b8": ("uniform_q4_0", 8, 32768, "uniform Q4_0 B=8 L=32768"),
    "uniform_q8_0_4k_b8": ("uniform_q8_0", 8, 4096, "uniform Q8_0 B=8 L=4096"),
    "uniform_f16_32k_b8": ("uniform_f16", 8, 32768, "uniform F16 B=8 L=32768"),
    "ragged_q4_0": ("ragged_q4_0", 8, 131072, "ragged Q4_0 131072+7x8192"),
    "ragged_small_q4_0": ("ragged_small_q4_0", 8, 4096, "ragged Q4_0 4096+7x256"),
    "tiny_f16": ("tiny_f16", 1, 200, "tiny F16 B=1 L=200"),
    "slab_f16": ("slab_f16", 8, 65536, "F16 D=128 Hq=32 Hkv=8 bs=32 B=8 L=65536, pool past 2^32 elements"),
}
# the batch sweeps of the uniform workloads (B = 1, 2, 4 next to the B = 8 rows above)
for _B in (1, 2, 4):
    WORKLOADS[f"uniform_q4_0_128k_b{_B}"] = ("uniform_q4_0", _B, 131072, f"uniform Q4_0 B={_B} L=131072")
    WORKLOADS[f"uniform_q4_0_32k_b{_B}"] = ("uniform_q4_0", _B, 32768, f"uniform Q4_0 B={_B} L=32768")
    WORKLOADS[f"uniform_q8_0_4k_b{_B}"] = ("uniform_q8_0", _B, 4096, f"uniform Q8_0 B={_B} L=4096")
SWEEP = [f"{w}_b{B}" for w in ("uniform_q8_0_4k", "uniform_q4_0_32k", "uniform_q4_0_128k")
         for B in (1, 2, 4, 8)]
DEFAULT = "uniform_q4_0_128k_b8"


DECODE_KERNELS = ("decode_kernel", "decode_lds_kernel")


def source_hash() -> str:
    """Hash of the decode kernels' sources: counter summaries taken on other
    sources are not used for `traffic`."""
    h = hashlib.sha256()
    for name in ("decode.hip", "decode_lds.hip", "lds_ring.h", "decode_common.h", "pa_device.h", "pa_host.h"):
        with open(os.path.join(ROOT, "paged_kv_gqa_attn_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(case, plan):
    """HBM bytes one step must move: live K/V rows, table entries, seq_len, q,
    partials (written by decode, read by merge) and out. Returns
    (decode_bytes, merge_bytes)."""
    import synth
    rbk = synth.row_bytes(case.k_fmt, case.D)
    rbv = synth.row_bytes(case.v_fmt, case.D)
    kv = sum(case.seq_lens) * case.Hkv * (rbk + rbv)
    table = sum(-(-L // case.block_size) for L in case.seq_lens) * 4
    q = 4 * case.B * case.Hq * case.D
    out = 4 * case.B * case.Hq * case.D
    seq = 4 * case.B
    if plan.direct:
        return kv + table + seq + q + out, 0
    parts = sum(-(-L // plan.psize) for L in case.seq_lens) * case.Hq * (2 * case.D + 8)
    return kv + table + seq + q + parts, parts + seq + out


def build_cases(name, seed, device, min_bytes):
    import synth
    wl, B, L, _ = WORKLOADS[name]
    first = synth.workload(wl, B=B, L=L, seed=seed, device=device, junk="zero")
    live = first.k_pool.numel() + first.v_pool.numel()
    copies = max(1, math.ceil(min_bytes / max(1, live)))
    if name == "slab_f16":
        copies = 1            # 18 GB of pools; its live rows (2.1 GB) already dwarf the MALL
    cases = [first] + [synth.workload(wl, B=B, L=L, seed=seed + 17 * i, device=device, junk="zero")
                       for i in range(1, copies)]
    return cases


def cpu_baseline(case, budget_s=20.0):
    """Time the fp64 oracle on a bounded sample of the workload: whole
    (sequence, kv-head) groups, in order, dealt over a thread pool of one
    worker per host core (at most 16, the CPU share of one GPU), each worker
    with one BLAS thread, until about budget_s of wall time."""
    from concurrent.futures import FIRST_COMPLETED, ThreadPoolExecutor, wait
    import oracle
    import synth
    from threadpoolctl import threadpool_limits
    host_cores = len(os.sched_getaffinity(0))
    workers = max(1, min(16, host_cores))
    kp = case.k_pool.cpu().numpy().reshape(-1)
    vp = case.v_pool.cpu().numpy().reshape(-1)
    tab = case.table.cpu()
    sl = case.seq_len.cpu()
    q = case.q.cpu()
    rbk, rbv = synth.row_bytes(case.k_fmt, case.D), synth.row_bytes(case.v_fmt, case.D)
    kw = dict(Hkv=case.Hkv, D=case.D, block_size=case.block_size, k_fmt=case.k_fmt,
              v_fmt=case.v_fmt, nblocks=case.nblocks, max_blocks=case.max_blocks, scale=case.scale)
    items = [(b, g) for b in range(case.B) for g in range(case.Hkv) if case.seq_lens[b] > 0]
    done = []
    t0 = time.perf_counter()
    cpu0 = time.process_time()
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        pending, nxt = {}, 0
        while nxt < len(items) or pending:
            while nxt < len(items) and len(pending) < workers and time.perf_counter() - t0 < budget_s:
                it = items[nxt]
                pending[ex.submit(oracle.decode_heads, q, kp, vp, tab, sl, items=[it], **kw)] = it
                nxt += 1
            if not pending:
                break
            fin, _ = wait(list(pending), return_when=FIRST_COMPLETED)
            for f in fin:
                f.result()
                done.append(pending.pop(f))
    wall = time.perf_counter() - t0
    busy = (time.process_time() - cpu0) / max(wall, 1e-9)
    nbytes = sum(case.seq_lens[b] * (rbk + rbv) for b, _ in done)
    toks = sum(case.seq_lens[b] for b, _ in done)
    return {
        "value": round(nbytes / wall / 1e9, 4),
        "unit": "GB/s",
        "cores": int(workers),
        "kind": "oracle",
        "host_cores": int(host_cores),
        "busy_cores": round(busy, 1),
        "blas_threads_per_worker": 1,
        "sample": (f"fp64 numpy oracle over {len(done)} of {len(items)} (sequence, kv-head) groups "
                   f"({toks} token rows, {nbytes} K/V bytes) in {wall:.1f} s on a pool of {workers} "
                   f"worker threads (one BLAS thread each; {busy:.1f} cores busy on average)"),
    }


def traffic_from_profiles(label):
    """Counter-measured HBM bytes per decode dispatch, if a summary for this
    workload exists and was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"decode_{label}_pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash():
        return None
    try:
        return int(float(kv["traffic_bytes_per_dispatch"]))
    except (KeyError, ValueError):
        return None


def run_bench(args):
    import torch
    import paged_kv_gqa_attn_amd as pa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    name = args.workload
    cases = build_cases(name, args.seed, dev, 4 * MALL_BYTES)
    c0 = cases[0]
    shape = pa.shape_of(c0.B, c0.Hq, c0.Hkv, c0.D, c0.block_size, c0.nblocks, c0.max_blocks,
                        c0.k_fmt, c0.v_fmt)
    plan = pa.paged_attn_plan(shape, max(c0.seq_lens), total_tokens=sum(c0.seq_lens),
                              force_partitions=args.force_partitions)
    if args.single_launch:
        plan.fused = 1
    ws = pa.workspace(plan, dev)
    out = torch.empty((c0.B, c0.Hq, c0.D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def step(c, ev_start=None, ev_end=None):
        if ev_start is not None:
            ev_start.record(stream)
        pa.paged_attn_decode(plan, c.q, c.k_pool, c.v_pool, c.table, c.seq_len, ws, out, stream=sptr)
        if ev_end is not None:
            ev_end.record(stream)
        pa.paged_attn_merge(plan, ws, c.seq_len, out, stream=sptr)

    # Clock settle: after idle the GPU's clocks take some tens of milliseconds
    # of sustained load to reach the level a serving loop runs at, so steps
    # run back to back for at least --settle-ms first (synchronising every 16
    # steps so the host never runs far ahead). Recorded in the JSON line.
    settle_steps, settle_t0 = 0, time.perf_counter()
    while (time.perf_counter() - settle_t0) * 1e3 < args.settle_ms:
        for _ in range(16):
            step(cases[settle_steps % len(cases)])
            settle_steps += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - settle_t0) * 1e3
    for i in range(args.warmup):
        step(cases[i % len(cases)])
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps with no event inside (an event
    # record costs the stream a few µs), bracketed by synchronisations.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(cases[i % len(cases)])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us_events = e0.elapsed_time(e1) * 1e3 / args.steps

    # Kernel split: the same steps again with two events per step around the
    # decode launch on its stream; the merge is timed from the decode's end
    # event to the next step's start event (one more event closes the loop).
    ev_start = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev_end = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        step(cases[i % len(cases)], ev_start[i], ev_end[i])
    ev_start[args.steps].record(stream)
    torch.cuda.synchronize()
    dec_ms = [ev_start[i].elapsed_time(ev_end[i]) for i in range(args.steps)]
    mrg_ms = [ev_end[i].elapsed_time(ev_start[i + 1]) for i in range(args.steps)]
    step_ms = [ev_start[i].elapsed_time(ev_start[i + 1]) for i in range(args.steps)]
    if pa.paged_attn_status(ws) != 0:
        raise SystemExit("bench: device status word set (bad table or seq_len)")

    dec_bytes, mrg_bytes = algorithmic_bytes(c0, plan)
    ms_per_step = wall * 1e3 / args.steps
    value = (dec_bytes + mrg_bytes) / (ms_per_step * 1e-3) / 1e9
    dec_avg = sum(dec_ms) / len(dec_ms)
    # a single-launch plan's decode kernel also reads the partials back and
    # writes out: all of the step's bytes are that one kernel's
    kern_bytes = dec_bytes + mrg_bytes if plan.fused else dec_bytes
    achieved = kern_bytes / (dec_avg * 1e-3) / 1e9
    med = sorted(step_ms)[len(step_ms) // 2]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": round(settle_ms, 1), "steps": settle_steps},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[name][3],
            "name": name,
            "B": c0.B, "Hq": c0.Hq, "Hkv": c0.Hkv, "D": c0.D, "block_size": c0.block_size,
            "k_type": c0.k_fmt, "v_type": c0.v_fmt, "seq_lens": sorted(set(c0.seq_lens)),
            "live_tokens": sum(c0.seq_lens), "psize": plan.psize, "p_max": plan.p_max,
            "grid": plan.grid, "decode_kernel": DECODE_KERNELS[plan.path - 1],
            "single_launch_merge": bool(plan.fused),
            "pool_copies": len(cases),
            "step_us_events": round(step_us_events, 2),
            "split_pass_step_us_median": round(med * 1e3, 2),
            "decode_us_mean": round(dec_avg * 1e3, 2),
            "merge_us_mean": round(sum(mrg_ms) / len(mrg_ms) * 1e3, 2),
            "step_pct_of_peak": round(100 * value / PEAK_GBS, 2),
            "algorithmic_bytes_per_step": dec_bytes + mrg_bytes,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4),
            "traffic": traffic_from_profiles(name),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(c0, budget_s=args.cpu_budget)
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# rocprofv3 summaries (text under profiles/)
# ---------------------------------------------------------------------------

def _csvs(d, suffix):
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def summarize_stats(d, label, cmd, stem=None):
    rows = []
    for path in _csvs(d, "kernel_stats.csv"):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    lines = [f"# rocprofv3 kernel statistics: {label}", f"# command: {cmd}",
             f"# source_hash = {source_hash()}",
             "# library kernels (the rest is the benchmark's input generation in torch)",
             "# name | calls | total_ns | average_ns | min_ns | max_ns | percent"]
    other_calls, other_ns = 0, 0
    for r in rows:
        nm = r.get("Name", r.get("KernelName", "?"))
        if "pa::" not in nm:
            other_calls += int(r.get("Calls", "0") or 0)
            other_ns += int(float(r.get("TotalDurationNs", "0") or 0))
            continue
        lines.append(" | ".join([nm[:110], r.get("Calls", ""), r.get("TotalDurationNs", ""),
                                 r.get("AverageNs", ""), r.get("MinNs", ""), r.get("MaxNs", ""),
                                 r.get("Percentage", "")]))
    lines.append(f"# other kernels: {other_calls} calls, {other_ns} ns in total")
    out = os.path.join(ROOT, "profiles", f"{stem or 'decode_' + label}_stats.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def summarize_pmc(d, label, cmd, calib_bytes):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the decode kernel, scaled
    by what the same counters read for the calibration copy of calib_bytes."""
    per = {}
    for path in _csvs(d, "counter_collection.csv"):
        with open(path) as f:
            for r in csv.DictReader(f):
                nm = r.get("Kernel_Name", "")
                cn = r.get("Counter_Name", "")
                val = float(r.get("Counter_Value", "0") or 0)
                did = r.get("Dispatch_Id", "")
                per.setdefault((nm, did), {}).setdefault(cn, 0.0)
                per[(nm, did)][cn] += val
    if not per:
        raise SystemExit(f"no counter_collection.csv under {d}")
    dec = [v for (nm, _), v in per.items() if any(k in nm for k in DECODE_KERNELS)]
    cpy = [v for (nm, _), v in per.items() if not any(k in nm for k in DECODE_KERNELS)
           and "merge" not in nm and "gather" not in nm]
    lines = [f"# rocprofv3 counters: {label}", f"# command: {cmd}", f"source_hash = {source_hash()}"]
    result = {}
    for cn in ("FETCH_SIZE", "WRITE_SIZE"):
        dv = [v[cn] for v in dec if cn in v]
        cv = [v[cn] for v in cpy if cn in v]
        if not dv:
            continue
        dec_kib = sum(dv) / len(dv)
        lines.append(f"decode_{cn}_KiB_per_dispatch = {dec_kib:.1f}")
        if cv:
            big = max(cv)
            factor = calib_bytes / (big * 1024.0)
            lines.append(f"calib_copy_{cn}_KiB = {big:.1f}  (copy of {calib_bytes} bytes)")
            lines.append(f"calib_factor_{cn} = {factor:.4f}")
            result[cn] = dec_kib * 1024.0 * factor
        else:
            result[cn] = dec_kib * 1024.0
    if result:
        tot = sum(result.values())
        lines.append(f"traffic_bytes_per_dispatch = {tot:.0f}")
    out = os.path.join(ROOT, "profiles", f"decode_{label}_pmc.txt")
    prev = []
    if os.path.exists(out):
        with open(out) as f:
            prev = [l.rstrip("\n") for l in f if l.startswith("decode_") or l.startswith("calib")]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def pmc_pass(args):
    """Counter pass: a calibration copy of known size, then a few decode steps."""
    import torch
    dev = torch.device("cuda:0")
    n = args.calib_bytes
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    args.no_cpu_baseline = True
    run_bench(args)


# name -> (synth workload, B, L, Tq, description)
CHUNKS = {
    "verify_q4_0_32k_b8_t8": ("uniform_q4_0", 8, 32768, 8, "verify window Q4_0 B=8 L=32768 Tq=8"),
    "verify_q4_0_32k_b8_t4": ("uniform_q4_0", 8, 32768, 4, "verify window Q4_0 B=8 L=32768 Tq=4"),
    "verify_q4_0_32k_b8_t2": ("uniform_q4_0", 8, 32768, 2, "verify window Q4_0 B=8 L=32768 Tq=2"),
    "prefill_q4_0_8k_t512": ("uniform_q4_0", 1, 8192, 512, "prefill chunk Q4_0 B=1 L=8192 Tq=512"),
    "verify_q4_0_d128_32k_b8_t8": ("uniform_q4_0_d128", 8, 32768, 8,
                                   "verify window Q4_0 D=128 Hq=32 Hkv=8 B=8 L=32768 Tq=8"),
}
PEAK_F16_TFLOPS = 2500.0   # MI355X dense f16 MFMA, public figure


def run_chunk(args):
    """Multi-token query (chunk) attention over the paged pool: one call of
    paged_attn_chunk (chunk kernel + merge) per step. Prints one JSON line with
    the step time, the algorithmic HBM bytes and the useful MFMA work (4*D
    flops per (query row, visible key)), each against its MI355X peak."""
    import torch
    import synth
    import paged_kv_gqa_attn_amd as pa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl, B, L, Tq, desc = CHUNKS[args.chunk]
    # pool copies rotated so that a step's K/V is not served from the MALL
    # (at most 16: a short prefill chunk's pool is small and stays hot anyway)
    cases = []
    need = 4 * MALL_BYTES
    while need > 0 and len(cases) < 16:
        c = synth.workload(wl, B=B, L=L, seed=args.seed + 17 * len(cases), device=dev, junk="zero")
        cases.append(c)
        need -= c.k_pool.numel() + c.v_pool.numel()
    c0 = cases[0]
    g = torch.Generator(device=dev).manual_seed(args.seed)
    qs = [torch.randn((B, Tq, c0.Hq, c0.D), generator=g, device=dev) for _ in cases]
    shape = pa.shape_of(c0.B, c0.Hq, c0.Hkv, c0.D, c0.block_size, c0.nblocks, c0.max_blocks,
                        c0.k_fmt, c0.v_fmt)
    plan = pa.paged_attn_chunk_plan(shape, Tq, L, total_tokens=B * L, force_partitions=args.force_partitions)
    if args.chunk_path:
        plan.path = args.chunk_path
    ws = pa.workspace(plan, dev)
    out = torch.empty((B, Tq, c0.Hq, c0.D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        c = cases[i % len(cases)]
        pa.paged_attn_chunk(plan, qs[i % len(cases)], c.k_pool, c.v_pool, c.table, c.seq_len, ws, out,
                            stream=stream)

    settle_steps, settle_t0 = 0, time.perf_counter()   # clock settle, as in run_bench
    while (time.perf_counter() - settle_t0) * 1e3 < args.settle_ms:
        for _ in range(16):
            step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - settle_t0) * 1e3
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall_us = (time.perf_counter() - t0) * 1e6 / args.steps
    gpu_us = e0.elapsed_time(e1) * 1e3 / args.steps
    if pa.paged_attn_status(ws) != 0:
        raise SystemExit("bench: device status word set")

    rb = synth.row_bytes(c0.k_fmt, c0.D) + synth.row_bytes(c0.v_fmt, c0.D)
    kv = B * L * c0.Hkv * rb
    rows = B * Tq * c0.Hq
    parts = 0 if plan.direct else rows * (-(-L // plan.psize)) * (2 * c0.D + 8) * 2
    nbytes = kv + B * (-(-L // c0.block_size)) * 4 + 2 * rows * c0.D * 4 + parts
    keys = B * c0.Hq * sum(L - Tq + t + 1 for t in range(Tq))
    flops = 4.0 * c0.D * keys
    gbs = nbytes / (wall_us * 1e-6) / 1e9
    tfs = flops / (wall_us * 1e-6) / 1e12
    hbm_frac, mfma_frac = gbs / PEAK_GBS, tfs / PEAK_F16_TFLOPS
    bound = "hbm" if hbm_frac >= mfma_frac else "mfma"
    line = {
        "metric": "paged chunk attention step (chunk kernel + merge)",
        "value": round(wall_us, 2), "unit": "us", "higher_is_better": False,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "settle": {"ms": round(settle_ms, 1), "steps": settle_steps}, "dtype": "f16", "data": "synthetic",
        "config": {"workload": desc, "name": args.chunk, "B": B, "L": L, "Tq": Tq, "Hq": c0.Hq,
                   "Hkv": c0.Hkv, "D": c0.D, "k_type": c0.k_fmt, "v_type": c0.v_fmt,
                   "psize": plan.psize, "p_max": plan.p_max, "grid": plan.grid,
                   "kernel": {1: "tile conversion", 2: "window", 3: "wide tile"}[plan.path],
                   "pool_copies": len(cases), "gpu_us_events": round(gpu_us, 2)},
        "roofline": {"bound": bound,
                     "hbm": {"achieved": round(gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
                             "frac": round(hbm_frac, 4), "bytes": nbytes},
                     "mfma": {"achieved": round(tfs, 1), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(mfma_frac, 4), "flops": flops}},
    }
    print(json.dumps(line), flush=True)


def run_metadata(args):
    """Paging-metadata maintenance (lucebox PR #555, Summary: only new blocks'
    ids are sent, not the table; Roadmap item 6: copy-on-write). Prints
    one JSON line:
      * table: paged_table_update of one fresh block per sequence plus its
        seq_len (the per-step upload at B=8, 16-token blocks, 128K-token
        tables), against copying the whole live table and seq_len from pinned
        host memory every step;
      * cow: paged_kv_copy_blocks of 64 1 MB blocks (256 slots x 8 heads of
        F16 D=256 rows) per call, rotating over a pool 5x the MALL, HBM bytes
        read + written per second.
    """
    import torch
    import paged_kv_gqa_attn_amd as pa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    B, MB, K = 8, 8192, max(args.steps, 20)

    def timed(fn, reps):
        for _ in range(5):
            fn(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / reps, e0.elapsed_time(e1) * 1e3 / reps

    table = torch.zeros((B, MB), dtype=torch.int32, device=dev)
    seq_len = torch.zeros(B, dtype=torch.int32, device=dev)
    host_table = torch.zeros((B, MB), dtype=torch.int32).pin_memory()
    host_seq = torch.zeros(B, dtype=torch.int32).pin_memory()

    def update(i):
        j = i % MB
        pa.paged_table_update(table, seq_len, [(b, j, b * MB + j) for b in range(B)] +
                              [(b, -1, 16 * (j + 1)) for b in range(B)], stream=stream)

    def full_upload(i):
        table.copy_(host_table, non_blocking=True)
        seq_len.copy_(host_seq, non_blocking=True)

    upd_wall, upd_gpu = timed(update, K)
    full_wall, full_gpu = timed(full_upload, K)

    # 1.25 GiB pool (5x the MALL); each call copies 64 blocks from the lower
    # half to the upper half, rotating so that no call finds its blocks cached
    nb, bsz = 1280, 256 * 8 * 512
    pool = torch.zeros((nb, 256, 8, 512), dtype=torch.uint8, device=dev)
    half = nb // 2

    def cow(i):
        base = (64 * i) % half
        src = [(base + k) % half for k in range(64)]
        dst = [half + (base + 320 + k) % half for k in range(64)]
        pa.paged_kv_copy_blocks(pool, src, dst, stream=stream)

    cow_wall, cow_gpu = timed(cow, K)
    cow_bytes = 2 * 64 * bsz
    line = {
        "metric": "paging metadata: per-step table update and copy-on-write block copy",
        "unit": "us",
        "n_gpus": 1,
        "steps": K,
        "data": "synthetic",
        "table": {"B": B, "max_blocks": MB, "update_entries": 2 * B,
                  "update_bytes": 2 * B * 12, "update_us_gpu": round(upd_gpu, 2),
                  "update_us_wall": round(upd_wall, 2),
                  "full_table_bytes": (B * MB + B) * 4, "full_upload_us_gpu": round(full_gpu, 2),
                  "full_upload_us_wall": round(full_wall, 2)},
        "cow": {"pairs": 64, "block_bytes": bsz, "us_gpu": round(cow_gpu, 2),
                "GB_s": round(cow_bytes / (cow_gpu * 1e-6) / 1e9, 1),
                "frac_of_8TBs": round(cow_bytes / (cow_gpu * 1e-6) / 1e9 / PEAK_GBS, 3)},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="back-to-back steps for at least this long before the warmup (recorded)")
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=1000)
    ap.add_argument("--force-partitions", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--single-launch", action="store_true",
                    help="decode and merge in one launch (plan.fused = 1; the planner's default is two)")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--pmc-pass", action="store_true")
    ap.add_argument("--calib-bytes", type=int, default=1 << 30)
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--summarize-pmc", metavar="DIR")
    ap.add_argument("--label", default=DEFAULT)
    ap.add_argument("--cmd", default="")
    ap.add_argument("--stem", default=None, help="profiles/ file stem (default decode_LABEL)")
    ap.add_argument("--chunk", default=None, choices=sorted(CHUNKS),
                    help="measure paged_attn_chunk on this workload instead of the decode step")
    ap.add_argument("--chunk-path", type=int, default=0, choices=[0, 1, 2, 3],
                    help="with --chunk: force the chunk kernel (1 tile conversion, 2 window, 3 wide tile)")
    ap.add_argument("--metadata", action="store_true",
                    help="measure the paging-metadata entry points instead of the decode step")
    ap.add_argument("--sweep", action="store_true",
                    help="one JSON line per workload of the batch sweep (no CPU baseline)")
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.label, args.cmd, args.stem)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.label, args.cmd, args.calib_bytes)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the decode step is measured at its one-GPU shape", file=sys.stderr)
        sys.exit(2)
    if args.pmc_pass:
        pmc_pass(args)
        return
    if args.metadata:
        run_metadata(args)
        return
    if args.chunk:
        run_chunk(args)
        return
    if args.sweep:
        args.no_cpu_baseline = True
        for name in SWEEP:
            args.workload = name
            run_bench(args)
        return
    run_bench(args)


if __name__ == "__main__":
    main()
