#!/usr/bin/env python3
"""Throughput of the varlen causal attention forward on one MI355X.

One step = one call of varlen_causal_attn_fwd (segment scheduler + attention
kernel) over the packed batch, with qkv and cu_seqlens already resident in HBM.
Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]
    python bench.py --mode bwd [--config 2]   # the training backward (varlen_causal_attn_bwd)

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
CSRC = os.path.join(ROOT, "varlen_causal_attention_amd", "csrc")
# The device sources each measured path runs (the profiles record their hash).
KERNEL_SOURCES = {
    "fwd": ("vlca_device.h", "vlca_order.h", "vlca_kernels.hip"),
    "bwd": ("vlca_device.h", "vlca_order.h", "vlca_kernels.hip", "vlca_backward.hip"),
    "masked": ("vlca_device.h", "vlca_order.h", "vlca_kernels.hip", "vlca_masked.hip"),
    "layer": ("vlca_device.h", "vlca_order.h", "vlca_kernels.hip", "vlca_proj.hip"),
}
ATTN_KERNEL = "attention_kernel"  # <true, true, false>: single-kernel plan; <false, ...>: over a worklist
PROFILE_PREFIX = {"fwd": "attention_kernel", "bwd": "backward", "masked": "masked_attention_kernel",
                  "layer": "attention_block"}


def kernel_source_hash(mode: str = "fwd") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[mode]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_name: str, mode: str = "fwd"):
    """HBM bytes per measured unit (the forward's attention kernel, or one backward
    call) from the committed rocprofv3 PMC summary, if it was taken on the current
    kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{PROFILE_PREFIX[mode]}_{workload_name}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(mode):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, budget_s: float, dout=None):
    """The fp64 oracle as it stands (the backward when ``dout`` is given), timed on
    this host over whole passes of the workload."""
    import numpy as np
    import torch

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = os.cpu_count() or 1
    q = w.qkv_bf16.to(torch.float64).numpy()
    d = None if dout is None else dout.to(torch.float64).numpy()
    passes = 0
    t0 = time.perf_counter()
    while True:
        if d is None:
            oracle.varlen_causal_attention(q, w.cu_seqlens, w.n_heads, w.head_dim, w.scale)
        else:
            oracle.varlen_causal_attention_backward(q, w.cu_seqlens, d, w.n_heads, w.head_dim, w.scale)
        passes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": passes * w.total_tokens / dt,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{passes} full pass(es) of the {'backward' if d is not None else 'forward'} over the {w.name} "
                  f"batch ({w.total_tokens} tokens, {w.num_users} users), fp64 numpy, {dt:.1f} s wall",
    }


# Counters of the SQ pass (eight SQ counters and one GRBM counter: within what
# one rocprofv3 pass can collect).
SQ_COUNTERS = ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32",
               "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_LDS", "GRBM_GUI_ACTIVE")

# Counters of the wait pass: where the waves' cycles go (waiting on counters or
# barriers, ready but not issued, issuing), in units of wave-cycles.
WAIT_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                 "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_SCA", "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE")

PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d {out}/trace -o run -- "
             "python3 {r}/bench.py --mode {m} --config {c} --steps 200 --warmup 2000 --no-cpu-baseline --cold-steps 0",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/fetch -o run -- "
             "python3 {r}/bench.py --mode {m} --config {c} --steps 5 --warmup 1 --no-cpu-baseline --cold-steps 0",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/write -o run -- "
             "python3 {r}/bench.py --mode {m} --config {c} --steps 5 --warmup 1 --no-cpu-baseline --cold-steps 0",
    "sq": "rocprofv3 --pmc " + " ".join(SQ_COUNTERS) + " --output-format csv -d {out}/sq -o run -- "
          "python3 {r}/bench.py --mode {m} --config {c} --steps 5 --warmup 1 --no-cpu-baseline --cold-steps 0",
    "waits": "rocprofv3 --pmc " + " ".join(WAIT_COUNTERS) + " --output-format csv -d {out}/waits -o run -- "
             "python3 {r}/bench.py --mode {m} --config {c} --steps 5 --warmup 1 --no-cpu-baseline --cold-steps 0",
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


def _short_name(name: str) -> str:
    m = re.search(r"([A-Za-z_]\w*(?:<[^>]*>)?)\(", name)
    return m.group(1) if m else name[:40]


def summarize_profiles(root: str, config: int, mode: str = "fwd") -> None:
    """Write profiles/<prefix>_<workload>_{trace,pmc,sq}.txt from rocprofv3 CSV output.

    ``root`` holds one folder per rocprofv3 run (commands in PROFILE_COMMANDS, with
    $REPO the repository root and $OUT the directory given to the runs, here
    ``root``; run from /tmp with TMPDIR=/tmp), plus ``kernel_sha.txt`` (the
    kernel_source_hash of the mode the runs used) and, optionally, ``trace.log``
    (that run's output with the bench line).  The prefix names the measured unit
    (PROFILE_PREFIX): the forward's attention kernel, the backward call, the
    masked kernel or the sub-block (counters: its LayerNorm + Linear_qkv product).
    """
    import workloads

    w = workloads.make_config(config, with_values=False)
    prefix = PROFILE_PREFIX[mode]
    sha_path = os.path.join(root, "kernel_sha.txt")
    sha = open(sha_path, encoding="utf-8").read().split()[0][:16] if os.path.exists(sha_path) else "unknown"
    if sha != kernel_source_hash(mode):
        print(f"warning: profiles were taken on kernel sources {sha}, tree has {kernel_source_hash(mode)}",
              file=sys.stderr)
    cmds = {k: "cd /tmp && export TMPDIR=/tmp && " + v.format(r="$REPO", out="$OUT", c=config, m=mode)
            for k, v in PROFILE_COMMANDS.items()}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    out_base = os.path.join(ROOT, "profiles", f"{prefix}_{w.name}")

    # Kernel trace: per-kernel duration statistics.
    stats = _read_csv(os.path.join(root, "trace", "run_kernel_stats.csv"))
    lines = [f"# rocprofv3 kernel trace, {mode} workload {w.name} ({w.total_tokens} tokens, {w.num_users} users)",
             f"# command: {cmds['trace']}",
             f"kernel_source_sha256_16: {sha}",
             "",
             f"{'kernel':<40} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}"]
    for r in stats:
        lines.append(f"{_short_name(r['Name']):<40} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>9.3f} "
                     f"{float(r['MinNs']) / 1e3:>9.3f} {float(r['MaxNs']) / 1e3:>9.3f} "
                     f"{float(r['Percentage']):>6.2f}")
    log = os.path.join(root, "trace.log")
    if os.path.exists(log):
        bench_lines = [ln for ln in open(log, encoding="utf-8") if ln.startswith("[bench]") or ln.startswith("{")]
        if bench_lines:
            lines += ["", "# the profiled bench run printed (its event timings include profiler overhead):"]
            lines += ["#   " + ln.rstrip()[:400] for ln in bench_lines]
    with open(out_base + "_trace.txt", "w", encoding="utf-8") as f:
        f.write("\n".join(lines) + "\n")

    # HBM traffic: FETCH_SIZE / WRITE_SIZE per dispatch, scaled by a plain copy's
    # reading.  Forward: the attention kernel that fwd runs.  Backward: the sum
    # over the kernels of one varlen_causal_attn_bwd call.
    fetch_rows = _read_csv(os.path.join(root, "fetch", "run_counter_collection.csv"))
    copy_f, _ = _counter_mean(os.path.join(root, "copyf"), COPY_KERNEL, "FETCH_SIZE")
    copy_w, _ = _counter_mean(os.path.join(root, "copyw"), COPY_KERNEL, "WRITE_SIZE")
    copy_bytes = 256 * 2**20
    f_factor = copy_bytes / (copy_f * 1024.0)
    w_factor = copy_bytes / (copy_w * 1024.0)
    if mode == "fwd":
        names = [n for n in (f"{ATTN_KERNEL}<true, true, false>", f"{ATTN_KERNEL}<false, true, false>",
                             f"{ATTN_KERNEL}<false, false, false>") if any(n in r["Kernel_Name"] for r in fetch_rows)]
        kernels = names[:1]
        algorithmic = w.algorithmic_bytes()
    elif mode == "masked":
        kernels = ["masked_attention_kernel"]
        algorithmic = w.algorithmic_bytes()
    elif mode == "layer":
        kernels = ["ln_proj_kernel"]
        algorithmic = ln_qkv_algorithmic_bytes(w.total_tokens)
    else:
        kernels = ["bwd_prepare_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"]
        algorithmic = backward_algorithmic_bytes(w)
    fetch_kib = write_kib = 0.0
    per = []
    for k in kernels:
        fk, n_f = _counter_mean(os.path.join(root, "fetch"), k, "FETCH_SIZE")
        wk, n_w = _counter_mean(os.path.join(root, "write"), k, "WRITE_SIZE")
        fetch_kib += fk
        write_kib += wk
        per.append(f"{k}: fetch_kib {fk:.3f} ({n_f} dispatches), write_kib {wk:.3f} ({n_w} dispatches)")
    rd = fetch_kib * 1024.0 * f_factor
    wr = write_kib * 1024.0 * w_factor
    lines = [f"# rocprofv3 HBM counters, {mode} workload {w.name}",
             f"# command (fetch): {cmds['fetch']}",
             f"# command (write): {cmds['write']}",
             f"# command (copy calibration, fetch): {cmds['copyf']}",
             f"# command (copy calibration, write): {cmds['copyw']}",
             "# FETCH_SIZE/WRITE_SIZE are KiB per dispatch; each is scaled by what it reads for a",
             "# 256 MiB device-to-device copy (known bytes), averaged over the dispatches listed.",
             f"kernel_source_sha256_16: {sha}",
             f"workload: {w.name}",
             f"kernels: {', '.join(kernels)}",
             *[f"# {x}" for x in per],
             f"fetch_kib_per_dispatch: {fetch_kib:.3f}",
             f"write_kib_per_dispatch: {write_kib:.3f}",
             f"copy_bytes: {copy_bytes}",
             f"copy_fetch_kib: {copy_f:.3f}",
             f"copy_write_kib: {copy_w:.3f}",
             f"fetch_scale: {f_factor:.4f}",
             f"write_scale: {w_factor:.4f}",
             f"hbm_read_bytes_per_launch: {rd:.0f}",
             f"hbm_write_bytes_per_launch: {wr:.0f}",
             f"hbm_bytes_per_launch: {rd + wr:.0f}",
             f"algorithmic_bytes_per_launch: {algorithmic}",
             f"traffic_over_algorithmic: {(rd + wr) / algorithmic:.4f}"]
    with open(out_base + "_pmc.txt", "w", encoding="utf-8") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))

    # SQ counters per kernel (per dispatch, averaged) and what they give.
    sq_dir = os.path.join(root, "sq")
    if os.path.exists(os.path.join(sq_dir, "run_counter_collection.csv")):
        rows = _read_csv(os.path.join(sq_dir, "run_counter_collection.csv"))
        acc = {}
        for r in rows:
            k = _short_name(r["Kernel_Name"])
            acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        simds = 4 * 256
        lines = [f"# rocprofv3 SQ counters, {mode} workload {w.name}: per-dispatch averages",
                 f"# command: {cmds['sq']}",
                 "# SQ_* are summed over the device's shader engines and XCDs; GRBM_GUI_ACTIVE is summed",
                 "# over the 8 XCDs, so GUI cycles of the dispatch = GRBM_GUI_ACTIVE / 8.",
                 "# mfma_busy_pct = SQ_VALU_MFMA_BUSY_CYCLES / (GUI cycles x 1024 SIMDs) x 100",
                 "# lds_bank_conflict_pct = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE x 100",
                 f"kernel_source_sha256_16: {sha}"]
        for k in sorted(acc):
            c = {n: sum(v) / len(v) for n, v in acc[k].items()}
            n = len(next(iter(acc[k].values())))
            lines.append("")
            lines.append(f"kernel: {k} ({n} dispatches)")
            for name in SQ_COUNTERS:
                if name in c:
                    lines.append(f"  {name}: {c[name]:.0f}")
            gui = c.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
            mf = c.get("SQ_INSTS_MFMA", 0.0)
            if gui > 0:
                lines.append(f"  gui_cycles: {gui:.0f}")
                lines.append(f"  mfma_busy_pct: {100.0 * c.get('SQ_VALU_MFMA_BUSY_CYCLES', 0.0) / (gui * simds):.2f}")
            if mf > 0:
                lines.append(f"  mfma_busy_cycles_per_mfma: {c.get('SQ_VALU_MFMA_BUSY_CYCLES', 0.0) / mf:.2f}")
                lines.append(f"  valu_per_mfma: {c.get('SQ_INSTS_VALU', 0.0) / mf:.2f}")
                lines.append(f"  trans_f32_per_mfma: {c.get('SQ_INSTS_VALU_TRANS_F32', 0.0) / mf:.3f}")
                lines.append(f"  lds_insts_per_mfma: {c.get('SQ_INSTS_LDS', 0.0) / mf:.3f}")
            if c.get("SQ_LDS_IDX_ACTIVE", 0.0) > 0:
                lines.append(f"  lds_bank_conflict_pct: "
                             f"{100.0 * c.get('SQ_LDS_BANK_CONFLICT', 0.0) / c['SQ_LDS_IDX_ACTIVE']:.3f}")
        with open(out_base + "_sq.txt", "w", encoding="utf-8") as f:
            f.write("\n".join(lines) + "\n")

    # Wait pass: per kernel, each counter as a share of the waves' cycles.
    wait_dir = os.path.join(root, "waits")
    if os.path.exists(os.path.join(wait_dir, "run_counter_collection.csv")):
        rows = _read_csv(os.path.join(wait_dir, "run_counter_collection.csv"))
        acc = {}
        for r in rows:
            k = _short_name(r["Kernel_Name"])
            acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        lines = [f"# rocprofv3 wait counters, {mode} workload {w.name}: per-dispatch averages",
                 f"# command: {cmds['waits']}",
                 "# SQ_WAIT_ANY: wave-cycles waiting on a counter (s_waitcnt) or a barrier; SQ_WAIT_INST_ANY:",
                 "# wave-cycles ready but not issued; SQ_ACTIVE_INST_*: wave-cycles issuing.  Shares are of",
                 "# SQ_WAVE_CYCLES (all resident waves' cycles).  mfma_busy is not in this pass (see _sq.txt).",
                 f"kernel_source_sha256_16: {sha}"]
        for k in sorted(acc):
            c = {n: sum(v) / len(v) for n, v in acc[k].items()}
            if not c.get("SQ_WAVE_CYCLES"):
                continue
            n = len(next(iter(acc[k].values())))
            lines.append("")
            lines.append(f"kernel: {k} ({n} dispatches)")
            for name in WAIT_COUNTERS:
                if name in c:
                    share = "" if name in ("GRBM_GUI_ACTIVE", "SQ_INSTS_MFMA", "SQ_WAVE_CYCLES") else \
                        f"  ({100.0 * c[name] / c['SQ_WAVE_CYCLES']:.1f}% of wave-cycles)"
                    lines.append(f"  {name}: {c[name]:.0f}{share}")
        with open(out_base + "_waits.txt", "w", encoding="utf-8") as f:
            f.write("\n".join(lines) + "\n")


def ln_qkv_algorithmic_bytes(T: int) -> int:
    """LayerNorm + Linear_qkv: x read, qkv written, W_qkv, gamma/beta and the bias read once."""
    return T * (512 + 1536) * 2 + 1536 * 512 * 2 + 2 * 512 * 2 + 1536 * 2


def out_residual_algorithmic_bytes(T: int) -> int:
    """Linear_out + bias + residual: attention output and residual read, y written, W_out and bias read once."""
    return T * (512 * 3) * 2 + 512 * 512 * 2 + 512 * 2


def backward_algorithmic_bytes(w) -> int:
    """qkv, out and dout read once, lse read once, dqkv written once."""
    hd = w.n_heads * w.head_dim
    return w.total_tokens * ((3 + 1 + 1 + 3) * hd * 2 + w.n_heads * 4)


# The pages' own figure for this path: their Triton varlen kernel took 0.111 ms on
# the 6,823-token / 60-user batch (cti2026 README page, FlashAttention_Varlen
# section; the hardware is not stated beside it, the deployment targets another
# GPU).  Another machine's number is context, not a baseline: vs_baseline is
# null and the ratio is reported as pages_ratio, on that batch only.
PAGES_6823_MS = 0.111


def pages_ratio(w, tokens_per_s):
    if w.total_tokens != 6823 or w.num_users != 60:
        return None
    return tokens_per_s / (w.total_tokens / (PAGES_6823_MS * 1e-3))


def roofline(flops: float, nbytes: float, seconds: float, traffic, kernel: str, **extra):
    """The roofline object: HBM-bound below the ridge (GB/s vs 8 TB/s), MFMA-bound above it."""
    if flops / nbytes < RIDGE:
        bound, achieved, peak, unit = "hbm", nbytes / seconds / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", flops / seconds / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
            "traffic": traffic, "kernel": kernel, "kernel_us": seconds * 1e6, "algorithmic_bytes": nbytes,
            "algorithmic_flops": flops, **extra}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # 2000 steps of the 6823-token batch are ~20 ms: measured step times settle
    # only after several ms of sustained load (with 20 warm-up steps the 44000-token
    # batch read 48.4 us, with 2000 42.7 us).
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (2 = 6823 tokens / 60 users)")
    ap.add_argument("--mode", choices=("fwd", "bwd", "masked", "layer"), default="fwd",
                    help="fwd: the forward (the default measurement); bwd: the training backward; "
                         "masked: the forward with an HSTU-style mask (MASK_RECIPE); layer: the attention "
                         "sub-block (LayerNorm + Linear_qkv, attention, Linear_out + residual)")
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
        summarize_profiles(args.summarize_profiles, args.config, args.mode)
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
    if args.mode == "bwd":
        run_backward(args, w, dev)
        return
    if args.mode == "masked":
        run_masked(args, w, dev)
        return
    if args.mode == "layer":
        run_layer(args, w, dev)
        return
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
    kernel_name = (f"{ATTN_KERNEL}<true, true, false>" if single
                   else f"{ATTN_KERNEL}<false, false, false> over a prebuilt worklist (fixed assignment)")
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
        "vs_baseline": None,
        "pages_ratio": pages_ratio(w, value),
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
        "roofline": roofline(flops, nbytes, ms_attn * 1e-3, traffic, kernel_name,
                             worklist_kernel_us=ms_worklist_kernel * 1e3),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(rec), flush=True)


# The masked forward's workload: HSTU-like users with up to 16 context tokens and
# up to 32 candidates in groups of 8, and a 256-token causal window (counts drawn
# per user from their own seeded generator).
MASK_RECIPE = {"contexts_max": 16, "targets_max": 32, "group": 8, "window": (256, 0), "seed": 7}


def mask_counts(w):
    import numpy as np

    rng = np.random.default_rng(MASK_RECIPE["seed"])
    c = rng.integers(0, MASK_RECIPE["contexts_max"] + 1, w.num_users)
    g = rng.integers(0, MASK_RECIPE["targets_max"] + 1, w.num_users)
    return c.astype(np.int32), g.astype(np.int32)


def visible_pairs(lengths, c, g, group, window) -> int:
    """Query-key pairs the mask admits, summed over users (counted row by row from
    the intervals of each row: context keys, windowed history, own candidate group)."""
    import numpy as np

    left, right = window
    assert right == 0
    total = 0
    for L, cu_, gu in zip(lengths, c, g):
        L = int(L)
        if L == 0:
            continue
        cc = min(max(int(cu_), 0), L)
        gg = min(max(int(gu), 0), L - cc)
        nc = L - gg
        i = np.arange(L)
        lo = np.maximum(cc, i - left) if left >= 0 else np.full(L, cc)
        hist = np.where(i >= cc, np.maximum(0, np.minimum(i, nc - 1) - lo + 1), 0)
        ctx = np.where(i < cc, cc, cc)
        gs = nc + ((i - nc) // group) * group
        grp = np.where(i >= nc, i - gs + 1, 0)
        total += int((ctx + hist + grp).sum())
    return total


def run_masked(args, w, dev):
    """One step = one varlen_causal_attn_fwd_masked call with MASK_RECIPE's per-user
    counts and window: the masked kernel alone on batches of the single-kernel
    plan, the scheduler and the masked kernel on larger ones."""
    import torch

    import varlen_causal_attention_amd as vlca

    qkv = w.qkv_bf16.to(dev)
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    c, g = mask_counts(w)
    ct, gt = torch.from_numpy(c).to(dev), torch.from_numpy(g).to(dev)
    out = torch.empty((w.total_tokens, w.n_heads * w.head_dim), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    rec = MASK_RECIPE

    def step():
        vlca.fwd_masked(qkv, cu, w.max_seqlen, num_contexts=ct, num_targets=gt, target_group_size=rec["group"],
                        window=rec["window"], n_heads=w.n_heads, scale=w.scale, out=out)

    print(f"[bench] masked {w.name}: T={w.total_tokens} U={w.num_users} recipe={rec}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    pairs = visible_pairs(w.lengths, c, g, rec["group"], rec["window"])
    flops = 4.0 * w.n_heads * w.head_dim * pairs
    nbytes = w.algorithmic_bytes()
    print(f"[bench] masked step {ms_step * 1e3:.2f} us, {pairs} visible pairs per head", file=sys.stderr, flush=True)
    value = w.total_tokens / (ms_step * 1e-3)
    print(json.dumps({
        "metric": "varlen masked attn fwd tokens/s + TFLOP/s (% bf16 MFMA peak), HSTU-style mask",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "total_tokens": w.total_tokens, "num_users": w.num_users,
                   "mask": {k: v for k, v in rec.items() if k != "seed"}, "visible_pairs_per_head": pairs},
        "tflops": flops / (ms_step * 1e-3) / 1e12,
        "pct_bf16_mfma_peak": 100.0 * flops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "roofline": roofline(flops, nbytes, ms_step * 1e-3, measured_traffic(w.name, "masked"),
                             "varlen_causal_attn_fwd_masked (masked_attention_kernel, after the scheduler on "
                             "batches past the single-kernel plan)"),
    }), flush=True)


def _time(step, args, stream):
    import torch

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / args.steps


def run_layer(args, w, dev):
    """One step = the layer's attention sub-block: varlen_causal_attn_ln_qkv
    (LayerNorm fused into the qkv product), varlen_causal_attn_fwd and
    varlen_causal_attn_out_residual (bias and residual fused into the output
    product), on synthetic layer parameters.  Each product is also timed alone;
    the roofline object is the qkv product's (the largest of the three)."""
    import torch

    import varlen_causal_attention_amd as vlca
    import workloads

    p = workloads.make_layer_params()
    gp = {k: getattr(p, k).to(dev) for k in ("gamma", "beta", "w_qkv", "b_qkv", "w_out", "b_out")}
    x = workloads.draw_layer_input(w.total_tokens).to(dev)
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    T = w.total_tokens
    qkv = torch.empty((T, 1536), dtype=torch.bfloat16, device=dev)
    attn = torch.empty((T, 512), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, 512), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def ln_step():
        vlca.ln_qkv(x, gp["gamma"], gp["beta"], gp["w_qkv"], gp["b_qkv"], eps=p.eps, out=qkv)

    def attn_step():
        vlca.fwd(qkv, cu, w.max_seqlen, scale=w.scale, out=attn)

    def out_step():
        vlca.out_residual(attn, gp["w_out"], gp["b_out"], x, out=y)

    def block():
        ln_step()
        attn_step()
        out_step()

    print(f"[bench] attention sub-block {w.name}: T={T}", file=sys.stderr, flush=True)
    ms_block = _time(block, args, stream)
    ms_ln = _time(ln_step, args, stream)
    ms_out = _time(out_step, args, stream)
    print(f"[bench] sub-block {ms_block * 1e3:.2f} us; ln_qkv {ms_ln * 1e3:.2f} us; out_residual "
          f"{ms_out * 1e3:.2f} us", file=sys.stderr, flush=True)
    f_qkv = 2.0 * T * 512 * 1536
    f_out = 2.0 * T * 512 * 512
    b_qkv = ln_qkv_algorithmic_bytes(T)
    b_out = out_residual_algorithmic_bytes(T)
    flops = f_qkv + w.causal_flops() + f_out
    value = T / (ms_block * 1e-3)
    print(json.dumps({
        "metric": "packed layer attention sub-block tokens/s (LayerNorm+Linear_qkv, attention, Linear_out+residual)",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_block, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random layer parameters)",
        "config": {"workload": w.name, "total_tokens": T, "num_users": w.num_users, "d_model": 512, "n_heads": 8},
        "tflops": flops / (ms_block * 1e-3) / 1e12,
        "ln_qkv_us": ms_ln * 1e3, "out_residual_us": ms_out * 1e3,
        "roofline": roofline(f_qkv, b_qkv, ms_ln * 1e-3, measured_traffic(w.name, "layer"),
                             "ln_proj_kernel (LayerNorm + Linear_qkv)"),
        "out_residual_roofline": roofline(f_out, b_out, ms_out * 1e-3, None,
                                          "res_proj_kernel (Linear_out + bias + residual)"),
    }), flush=True)


def run_backward(args, w, dev):
    """One step = one varlen_causal_attn_bwd call (worklist and row pass in one kernel, dK/dV and
    dQ kernels) over the batch, with qkv, out, dout and lse resident in HBM."""
    import torch

    import varlen_causal_attention_amd as vlca
    import workloads

    qkv = w.qkv_bf16.to(dev)
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    dout_cpu = workloads.draw_dout(w.total_tokens, w.n_heads, seed=1)
    dout = dout_cpu.to(dev)
    out, lse = vlca.fwd_lse(qkv, cu, w.max_seqlen, n_heads=w.n_heads, scale=w.scale)
    dqkv = torch.empty_like(qkv)
    stream = torch.cuda.current_stream(dev)

    def step():
        vlca.bwd(qkv, out, dout, lse, cu, w.max_seqlen, n_heads=w.n_heads, scale=w.scale, dqkv=dqkv)

    print(f"[bench] backward {w.name}: T={w.total_tokens} U={w.num_users} max_seqlen={w.max_seqlen} "
          f"warmup={args.warmup} steps={args.steps}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] backward step {ms_step * 1e3:.2f} us", file=sys.stderr, flush=True)
    # Algorithmic work: the four products dV = P^T dO, dP = dO V^T, dQ = dS K and
    # dK = dS^T Q over the causal triangle (twice the forward's two); bytes: qkv,
    # out, dout and lse read once, dqkv written once.
    flops = 2.0 * w.causal_flops()
    nbytes = backward_algorithmic_bytes(w)
    value = w.total_tokens / (ms_step * 1e-3)
    rec = {
        "metric": "varlen causal attn bwd tokens/s + TFLOP/s (% bf16 MFMA peak)",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "total_tokens": w.total_tokens, "num_users": w.num_users,
                   "max_seqlen": w.max_seqlen, "n_heads": w.n_heads, "head_dim": w.head_dim,
                   "pass": "backward (dq, dk, dv from dout, out, lse)"},
        "tflops": flops / (ms_step * 1e-3) / 1e12,
        "pct_bf16_mfma_peak": 100.0 * flops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "roofline": roofline(flops, nbytes, ms_step * 1e-3, measured_traffic(w.name, "bwd"),
                             "varlen_causal_attn_bwd (prepare, dK/dV and dQ kernels)"),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_budget, dout=dout_cpu)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
