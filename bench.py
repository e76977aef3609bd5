#!/usr/bin/env python3
"""Throughput of the varlen causal attention forward on one MI355X.

One step = one call of varlen_causal_attn_fwd (segment scheduler + attention
kernel) over the packed batch, with qkv and cu_seqlens already resident in HBM.
Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]

The default workload is the pages' size: 6823 packed tokens over 60 users,
8 heads x 64, bf16 qkv [6823, 1536] (synthetic, seeded; see workloads.py).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
KERNEL_SRC = os.path.join(ROOT, "varlen_causal_attention_amd", "csrc", "vlca_kernels.hip")
ATTN_KERNEL = "attention_kernel"           # <true, true>: single-kernel plan; <false, ...>: over a worklist


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload_name: str):
    """HBM bytes per attention launch from the committed rocprofv3 PMC summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"attention_kernel_{workload_name}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle as it stands, timed on this host over whole passes of the workload."""
    import numpy as np
    import torch

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = os.cpu_count() or 1
    q = w.qkv_bf16.to(torch.float64).numpy()
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.varlen_causal_attention(q, w.cu_seqlens, w.n_heads, w.head_dim, w.scale)
        passes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": passes * w.total_tokens / dt,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{passes} full pass(es) of the {w.name} batch ({w.total_tokens} tokens, {w.num_users} users), "
                  f"fp64 numpy, {dt:.1f} s wall",
    }


PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d {out}/trace -o run -- "
             "python3 {r}/bench.py --config {c} --steps 200 --warmup 2000 --no-cpu-baseline --cold-steps 0",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/fetch -o run -- "
             "python3 {r}/bench.py --config {c} --steps 5 --warmup 1 --no-cpu-baseline --cold-steps 0",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/write -o run -- "
             "python3 {r}/bench.py --config {c} --steps 5 --warmup 1 --no-cpu-baseline --cold-steps 0",
    "copyf": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/copyf -o run -- "
             "python3 {r}/bench.py --calibrate-copy-mib 256 --steps 5",
    "copyw": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/copyw -o run -- "
             "python3 {r}/bench.py --calibrate-copy-mib 256 --steps 5",
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _read_csv(path):
    import csv

    with open(path, newline="", encoding="utf-8") as f:
        return list(csv.DictReader(f))


def _counter_mean(d: str, kernel_substr: str, counter: str):
    rows = [r for r in _read_csv(os.path.join(d, "run_counter_collection.csv"))
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    vals = [float(r["Counter_Value"]) for r in rows]
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel_substr} under {d}")
    return sum(vals) / len(vals), len(vals)


def summarize_profiles(root: str, config: int) -> None:
    """Write profiles/attention_kernel_<workload>_{trace,pmc}.txt from rocprofv3 CSV output.

    ``root`` holds one folder per rocprofv3 run (commands in PROFILE_COMMANDS, with
    $REPO the repository root and $OUT the directory given to the runs, here
    ``root``; run from /tmp with TMPDIR=/tmp), plus
    ``kernel_sha.txt`` (sha256 of the kernel source the runs used) and, optionally,
    ``trace.log`` (that run's stdout/stderr with the bench line).
    """
    import workloads

    w = workloads.make_config(config, with_values=False)
    sha_path = os.path.join(root, "kernel_sha.txt")
    sha = open(sha_path, encoding="utf-8").read().split()[0][:16] if os.path.exists(sha_path) else "unknown"
    if sha != kernel_source_hash():
        print(f"warning: profiles were taken on kernel source {sha}, tree has {kernel_source_hash()}",
              file=sys.stderr)
    cmds = {k: "cd /tmp && export TMPDIR=/tmp && " + v.format(r="$REPO", out="$OUT", c=config)
            for k, v in PROFILE_COMMANDS.items()}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)

    # Kernel trace: per-kernel duration statistics.
    stats = _read_csv(os.path.join(root, "trace", "run_kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel trace, workload {w.name} ({w.total_tokens} tokens, {w.num_users} users)",
             f"# command: {cmds['trace']}",
             f"kernel_source_sha256_16: {sha}",
             "",
             f"{'kernel':<28} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}"]
    for r in stats:
        m = re.search(r"([A-Za-z_]\w*(?:<[^>]*>)?)\(", r["Name"])
        short = m.group(1) if m else r["Name"][:28]
        lines.append(f"{short:<28} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>9.3f} "
                     f"{float(r['MinNs']) / 1e3:>9.3f} {float(r['MaxNs']) / 1e3:>9.3f} "
                     f"{float(r['Percentage']):>6.2f}")
    log = os.path.join(root, "trace.log")
    if os.path.exists(log):
        bench_lines = [ln for ln in open(log, encoding="utf-8") if ln.startswith("[bench]") or ln.startswith("{")]
        if bench_lines:
            lines += ["", "# the profiled bench run printed (its event timings include profiler overhead):"]
            lines += ["#   " + ln.rstrip()[:400] for ln in bench_lines]
    with open(os.path.join(ROOT, "profiles", f"attention_kernel_{w.name}_trace.txt"), "w", encoding="utf-8") as f:
        f.write("\n".join(lines) + "\n")

    # HBM traffic: FETCH_SIZE / WRITE_SIZE per dispatch, scaled by a plain copy's reading,
    # for the attention kernel fwd runs (the single-kernel instance when present).
    fetch_rows = _read_csv(os.path.join(root, "fetch", "run_counter_collection.csv"))
    kern = f"{ATTN_KERNEL}<true, true>" if any(f"{ATTN_KERNEL}<true, true>" in r["Kernel_Name"] for r in fetch_rows) \
        else f"{ATTN_KERNEL}<false"
    fetch_kib, n_f = _counter_mean(os.path.join(root, "fetch"), kern, "FETCH_SIZE")
    write_kib, n_w = _counter_mean(os.path.join(root, "write"), kern, "WRITE_SIZE")
    copy_f, _ = _counter_mean(os.path.join(root, "copyf"), COPY_KERNEL, "FETCH_SIZE")
    copy_w, _ = _counter_mean(os.path.join(root, "copyw"), COPY_KERNEL, "WRITE_SIZE")
    copy_bytes = 256 * 2**20
    f_factor = copy_bytes / (copy_f * 1024.0)
    w_factor = copy_bytes / (copy_w * 1024.0)
    rd = fetch_kib * 1024.0 * f_factor
    wr = write_kib * 1024.0 * w_factor
    lines = [f"# rocprofv3 HBM counters for {kern}, workload {w.name}",
             f"# command (fetch): {cmds['fetch']}",
             f"# command (write): {cmds['write']}",
             f"# command (copy calibration, fetch): {cmds['copyf']}",
             f"# command (copy calibration, write): {cmds['copyw']}",
             "# FETCH_SIZE/WRITE_SIZE are KiB per dispatch; each is scaled by what it reads for a",
             "# 256 MiB device-to-device copy (known bytes), averaged over the dispatches listed.",
             f"kernel_source_sha256_16: {sha}",
             f"workload: {w.name}",
             f"kernel: {kern}",
             f"fetch_kib_per_dispatch: {fetch_kib:.3f}",
             f"fetch_dispatches: {n_f}",
             f"write_kib_per_dispatch: {write_kib:.3f}",
             f"write_dispatches: {n_w}",
             f"copy_bytes: {copy_bytes}",
             f"copy_fetch_kib: {copy_f:.3f}",
             f"copy_write_kib: {copy_w:.3f}",
             f"fetch_scale: {f_factor:.4f}",
             f"write_scale: {w_factor:.4f}",
             f"hbm_read_bytes_per_launch: {rd:.0f}",
             f"hbm_write_bytes_per_launch: {wr:.0f}",
             f"hbm_bytes_per_launch: {rd + wr:.0f}",
             f"algorithmic_bytes_per_launch: {w.algorithmic_bytes()}",
             f"traffic_over_algorithmic: {(rd + wr) / w.algorithmic_bytes():.4f}"]
    with open(os.path.join(ROOT, "profiles", f"attention_kernel_{w.name}_pmc.txt"), "w", encoding="utf-8") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# The pages' own figure for this path: their Triton varlen kernel took 0.111 ms on
# the 6,823-token / 60-user batch (cti2026 README page, FlashAttention_Varlen
# section; the hardware is not stated beside it).  It is context, not a target:
# vs_baseline is the ratio of this build's tokens/s to that figure's, on that
# batch only.
PAGES_6823_MS = 0.111


def vs_baseline(w, tokens_per_s):
    if w.total_tokens != 6823 or w.num_users != 60:
        return None
    return tokens_per_s / (w.total_tokens / (PAGES_6823_MS * 1e-3))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # 2000 steps of the 6823-token batch are ~20 ms: measured step times settle
    # only after several ms of sustained load (with 20 warm-up steps the 44000-token
    # batch read 48.4 us, with 2000 42.7 us).
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (2 = 6823 tokens / 60 users)")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB --steps times (HBM counter calibration)")
    ap.add_argument("--cold-steps", type=int, default=30,
                    help="single launches timed after a 512 MiB scratch write (cache-cold step time)")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="no GPU: turn the rocprofv3 CSV output under DIR (trace/, fetch/, write/, copyf/, "
                         "copyw/) into the text summaries under profiles/")
    args = ap.parse_args()

    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.config)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(users would shard across GPUs with no exchange between them).", file=sys.stderr)
        sys.exit(2)

    import torch

    import varlen_causal_attention_amd as vlca
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * 2**20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                          "launches": args.steps}), flush=True)
        return
    w = workloads.make_config(args.config)
    qkv = w.qkv_bf16.to(dev)
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    out = torch.empty((w.total_tokens, w.n_heads * w.head_dim), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        vlca.fwd(qkv, cu, w.max_seqlen, n_heads=w.n_heads, head_dim=w.head_dim, scale=w.scale, out=out)

    print(f"[bench] {w.name}: T={w.total_tokens} U={w.num_users} max_seqlen={w.max_seqlen} "
          f"warmup={args.warmup} steps={args.steps}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Whole hot path: K steps back to back between two events on the launch stream.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps

    # Dominant kernel.  When fwd is a single kernel (small batches), the K steps
    # above are K launches of it back to back: its duration is the step time.
    # Otherwise the attention kernel alone over a prebuilt worklist, launched back
    # to back on the same stream, timed with events on that stream.
    single = vlca.single_kernel(w.num_users, w.max_seqlen, w.n_heads)
    items, _count = vlca.build_worklist(cu, w.max_seqlen)
    for _ in range(args.warmup):
        vlca.fwd_with_worklist(qkv, cu, w.max_seqlen, items, _count, scale=w.scale, out=out)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        vlca.fwd_with_worklist(qkv, cu, w.max_seqlen, items, _count, scale=w.scale, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_worklist_kernel = e0.elapsed_time(e1) / args.steps
    ms_attn = ms_step if single else ms_worklist_kernel
    kernel_name = f"{ATTN_KERNEL}<true, true>" if single else f"{ATTN_KERNEL}<false, ...>"
    print(f"[bench] step {ms_step * 1e3:.2f} us ({'single kernel' if single else 'scheduler + attention'}), "
          f"attention kernel over a worklist {ms_worklist_kernel * 1e3:.2f} us", file=sys.stderr, flush=True)

    # Cache-cold step: a 512 MiB write evicts L2 and the 256 MiB MALL before each
    # single timed step.
    cold_ms = None
    if args.cold_steps > 0:
        scratch = torch.empty(512 * 2**20, dtype=torch.uint8, device=dev)
        cold = []
        for _ in range(args.cold_steps):
            scratch.fill_(1)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del scratch
        cold_ms = sorted(cold)[len(cold) // 2]

    flops = w.causal_flops()
    nbytes = w.algorithmic_bytes()
    tflops = flops / (ms_step * 1e-3) / 1e12
    ai = flops / nbytes
    if ai < RIDGE:
        bound, achieved, peak, unit = "hbm", nbytes / (ms_attn * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", flops / (ms_attn * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    traffic = measured_traffic(w.name)

    value = w.total_tokens / (ms_step * 1e-3)
    rec = {
        "metric": "varlen causal attn fwd tokens/s + TFLOP/s (% bf16 MFMA peak), 6823tok/60users",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": vs_baseline(w, value),
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "total_tokens": w.total_tokens,
            "num_users": w.num_users,
            "max_seqlen": w.max_seqlen,
            "n_heads": w.n_heads,
            "head_dim": w.head_dim,
            "qkv": f"bf16 [{w.total_tokens}, {3 * w.n_heads * w.head_dim}]",
            "length_law": "lognormal(4.3, 0.9) rescaled, seed 0" if args.config == 2 else "see workloads.py",
            "launch": "single kernel" if single else "scheduler + attention kernel",
        },
        "cold_ms_per_step": cold_ms,
        "tflops": tflops,
        "pct_bf16_mfma_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "causal_gflop": flops / 1e9,
        "roofline": {
            "bound": bound,
            "achieved": achieved,
            "peak": peak,
            "unit": unit,
            "frac": achieved / peak,
            "traffic": traffic,
            "kernel": kernel_name,
            "kernel_us": ms_attn * 1e3,
            "worklist_kernel_us": ms_worklist_kernel * 1e3,
            "algorithmic_bytes": nbytes,
            "algorithmic_flops": flops,
        },
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
