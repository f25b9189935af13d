#!/usr/bin/env python3
"""Benchmark: batch-invariant paged-attention decode on one MI355X.

A step is one decode step of the Llama-3-8B-shaped workload (32 query / 8 KV heads, head_dim
128, bf16 pages of 16 tokens, fixed 2048-token splits, contexts uniform in [512, 8192], batch
256): the step's new K/V rows are written into their page slots (kv_append) and every
sequence's query row attends its whole paged context (decode split kernel + ascending split
merge).  The timed region starts with every input resident in HBM.

`value` is decode KV-read throughput: the algorithmic KV bytes of a step (sum_b n_b * Hkv * d *
2 tensors * 2 bytes -- each sequence's K and V read once per KV head) divided by the step time
(K steps timed between two device synchronisations).  The JSON line also carries:
  - roofline: the decode call's own duration from HIP events on the launch stream, with the HBM
    traffic of the split kernel from the committed rocprofv3 counters;
  - references: a plain streaming-read kernel (the achievable-HBM reference), torch's device copy
    and sum, and kv_append at prefill size (32768 rows);
  - batch sizes 1/8/64/256 (steady state and caches flushed), the split-by-count variant under the
    automatic kernel choice and with the split kernel pinned for both policies (the cost of
    invariance on one kernel), the bitwise-equivalent decode kernels at small batches;
  - a bitwise invariance rate over execution variations measured in the same run;
  - Qwen3-8B prefill: whole, in chunks of 64/256/1024, and over a cached 2048-token prefix;
  - Qwen3-235B-shaped decode at 32768 context, batch 1/16/64, and the mixed decode + prefill batch;
  - Llama-3.1-70B-shaped decode on a 16384-token shared prefix (bf16 and fp8), and one 131072-key
    sequence;
  - the batch-invariant layer operators against the vendor library;
  - the fp64 CPU oracle on the whole headline workload (all host threads) and single-thread
    figures for the tiny decode and for 8 sequences;
  - a manifest (git commit, source hash, gfx architecture, config hash).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
    python bench.py --decode-only ...   headline decode only (for profilers)
    python bench.py --copy-probe        a plain copy of known size (counter calibration)
    python bench.py --summarize-profile TRACE_DIR PMC_DIR   write the profile summary under profiles/
    python bench.py --summarize-spread-profile TRACE_DIR    the batch-1 spread-kernel trace summary
    python bench.py --summarize-layer-profile TRACE_DIR LAYER_JSON   the layer-operator trace summary

The roofline's `traffic` (HBM bytes per launch of the decode split kernel) comes from rocprofv3
FETCH_SIZE / WRITE_SIZE counters, each scaled by what the same counter reads for a plain 1 GiB
device copy; the figures live in profiles/ with the source hash of the kernel they were taken on,
and `traffic` is null whenever the kernel's sources have changed since.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import re
import math
import os
import subprocess
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from invariant_attention_amd import binding as ia  # noqa: E402
from synth import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
DEV = "cuda"
SEED = 0
COPY_PROBE_BYTES = 1 << 30
PROFILE_MD = os.path.join(ROOT, "profiles", "decode_split_kernel_llama3-8b_b256.md")
PREFILL_PROFILE_MD = os.path.join(ROOT, "profiles", "prefill_kernel_qwen3-8b_8x4096.md")
MFMA_FLOPS = 16 * 16 * 32 * 2  # one v_mfma_f32_16x16x32_bf16 of one wave
KERNEL_SOURCES = ["decode.hip", "arith.hpp", "pages.hpp", "launch.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def git_sha():
    try:
        return subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True, text=True,
                              timeout=10).stdout.strip() or None
    except Exception:
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def kernel_source_hash() -> str:
    """sha256 (first 16 hex digits) of the decode kernel's sources."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "invariant_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per decode_split_kernel launch recorded in profiles/, if taken on these sources."""
    try:
        text = open(PROFILE_MD).read()
    except OSError:
        return None
    rec = {}
    for line in text.splitlines():
        if line.startswith("traffic_record:"):
            rec = dict(kv.split("=", 1) for kv in line.split(":", 1)[1].split())
    if rec.get("source_sha") != kernel_source_hash():
        return None
    return int(rec["bytes_per_launch"])


def _csv_rows(pattern):
    rows = []
    for path in glob.glob(pattern, recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _pmc_mean(pmc_dir, kind, counter, kernel):
    """Mean per dispatch of one counter for one kernel, from the run in <pmc_dir>/pmc_<kind>_<counter>
    (a run may hold several counters; the directory is named for the first)."""
    rows = _csv_rows(os.path.join(pmc_dir, f"pmc_{kind}_{counter}", "**", "*counter_collection.csv"))
    if not rows:
        rows = _csv_rows(os.path.join(pmc_dir, f"pmc_{kind}_*", "**", "*counter_collection.csv"))
    vals = [float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter]
    return (float(np.mean(vals)) if vals else float("nan")), len(vals)


SPLIT_KERNEL = "decode_split_kernel<128, false"  # bf16 pages, either load policy
SHARED_PREFIX_PROFILE_MD = os.path.join(ROOT, "profiles", "decode_split_kernel_llama70b_shared_prefix.md")


def _decode_profile_lines(trace_dir, pmc_dir, kind, alg, title, workload, bench_args, pmc_steps):
    """Kernel-trace stats and calibrated FETCH/WRITE bytes of the decode split kernel for one workload.
    Returns (markdown lines, HBM bytes read per launch, written per launch, mean ns per launch)."""
    stats = _csv_rows(os.path.join(trace_dir, "**", "*kernel_stats.csv"))
    split = [r for r in stats if SPLIT_KERNEL in r["Name"]]
    merge = [r for r in stats if "decode_merge_kernel<128, false>" in r["Name"]]
    order = [r for r in stats if "decode_order_kernel" in r["Name"]]
    avg_ns = float(split[0]["AverageNs"])
    fetch_kib, nf = _pmc_mean(pmc_dir, kind, "FETCH_SIZE", SPLIT_KERNEL)
    write_kib, nw = _pmc_mean(pmc_dir, kind, "WRITE_SIZE", SPLIT_KERNEL)
    copy_fetch, _ = _pmc_mean(pmc_dir, "copy", "FETCH_SIZE", "__amd_rocclr_copyBuffer")
    copy_write, _ = _pmc_mean(pmc_dir, "copy", "WRITE_SIZE", "__amd_rocclr_copyBuffer")
    f_scale = COPY_PROBE_BYTES / (copy_fetch * 1024)
    w_scale = COPY_PROBE_BYTES / (copy_write * 1024)
    fetch_b = fetch_kib * 1024 * f_scale
    write_b = write_kib * 1024 * w_scale
    cmd_trace = (f"rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o {kind} -- "
                 f"python3 bench.py {bench_args} --steps 10 --warmup 3 --no-cpu-baseline")
    cmd_pmc = ("rocprofv3 --pmc {C} --output-format csv -d <out> -o pmc -- "
               f"python3 bench.py {bench_args} --steps {pmc_steps} --warmup 1 --no-cpu-baseline")
    cmd_copy = "rocprofv3 --pmc {C} --output-format csv -d <out> -o pmc -- python3 bench.py --copy-probe --steps 3"
    lines = [f"# {title}", "", workload, "", "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
             f"    {cmd_trace}", "", "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in order + split + merge:
        lines.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")
    lines += [
        "",
        f"Achieved from the trace: {alg / avg_ns:.1f} GB/s of algorithmic KV bytes = "
        f"{alg / avg_ns / HBM_PEAK_GBS:.4f} of the 8 TB/s HBM peak (split kernel alone; the dispatch-order "
        "kernel before it and the split merge after it add a few us each per call).",
        "",
        "## HBM traffic (rocprofv3 --pmc, one counter per run)",
        "",
        f"    {cmd_pmc.format(C='FETCH_SIZE')}",
        f"    {cmd_pmc.format(C='WRITE_SIZE')}",
        f"    {cmd_copy.format(C='FETCH_SIZE')}",
        f"    {cmd_copy.format(C='WRITE_SIZE')}",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| FETCH_SIZE per decode_split_kernel dispatch (KiB, mean of {nf}) | {fetch_kib:.1f} |",
        f"| WRITE_SIZE per decode_split_kernel dispatch (KiB, mean of {nw}) | {write_kib:.1f} |",
        f"| FETCH_SIZE of a 1 GiB device copy (KiB) | {copy_fetch:.1f} |",
        f"| WRITE_SIZE of a 1 GiB device copy (KiB) | {copy_write:.1f} |",
        f"| fetch scale (bytes read / counter bytes) | {f_scale:.4f} |",
        f"| write scale | {w_scale:.4f} |",
        f"| HBM bytes read per launch | {fetch_b:.4e} |",
        f"| HBM bytes written per launch | {write_b:.4e} |",
        f"| traffic / algorithmic bytes | {(fetch_b + write_b) / alg:.4f} |",
        f"| DRAM-side rate (HBM bytes read / kernel time) | {fetch_b / avg_ns:.1f} GB/s = "
        f"{fetch_b / avg_ns / HBM_PEAK_GBS:.4f} of peak |",
        "",
    ]
    hit, nh = _pmc_mean(pmc_dir, kind, "TCC_HIT_sum", SPLIT_KERNEL)
    miss, _ = _pmc_mean(pmc_dir, kind, "TCC_MISS_sum", SPLIT_KERNEL)
    if nh:
        lines += [
            "## L2 (rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum, one run)",
            "",
            f"    {cmd_pmc.format(C='TCC_HIT_sum TCC_MISS_sum')}",
            "",
            "| quantity | value |",
            "|---|---|",
            f"| TCC_HIT_sum per dispatch (mean of {nh}) | {hit:.4e} |",
            f"| TCC_MISS_sum per dispatch | {miss:.4e} |",
            f"| L2 hit rate | {hit / (hit + miss):.4f} |",
            "",
        ]
    return lines, fetch_b, write_b, avg_ns


def summarize_profile(trace_dir, pmc_dir):
    """Writes the headline decode profile summary (rocprofv3 kernel-trace stats + calibrated FETCH/WRITE)
    and the traffic record the bench's roofline reads."""
    lens = wl.uniform_lens(SEED, 256, 512, 8192)
    alg = int(sum(lens)) * 8 * 128 * 2 * 2
    lines, fetch_b, write_b, _ = _decode_profile_lines(
        trace_dir, pmc_dir, "decode", alg,
        "decode_split_kernel<128, bf16> -- Llama-3-8B-shaped decode, batch 256, contexts U[512, 8192]",
        "32 query / 8 KV heads, head_dim 128, bf16 pages of 16 tokens, fixed 2048-token splits, "
        f"{int(sum(lens))} context tokens; algorithmic KV bytes per launch {alg} "
        "(sum_b n_b x 8 heads x 128 dims x 2 tensors x 2 bytes).  The launch has ~5.3k split units, so the "
        "automatic cache hint streams its K/V loads (nontemporal).",
        "--decode-only", 3)
    tr = int(round(fetch_b + write_b))
    lines += [
        "The K/V stream is read once; the few L2 hits are block-table, query and split-partial reads.",
        "",
        f"traffic_record: source_sha={kernel_source_hash()} bytes_per_launch={tr} read={int(fetch_b)} "
        f"write={int(write_b)} algorithmic={alg}",
        "",
    ]
    os.makedirs(os.path.dirname(PROFILE_MD), exist_ok=True)
    with open(PROFILE_MD, "w") as f:
        f.write("\n".join(lines))
    print(PROFILE_MD)


def _shared_prefix_lens():
    rng = np.random.default_rng([SEED, 5])
    return [16384 + int(x) for x in rng.integers(256, 4097, 128)]


def summarize_shared_prefix_profile(trace_dir, pmc_dir):
    """Writes the Llama-3.1-70B shared-prefix decode profile: logical KV bytes against the DRAM bytes
    that FETCH_SIZE counts for the same launch."""
    shape = wl.LLAMA31_70B
    lens = _shared_prefix_lens()
    alg = int(sum(lens)) * shape.Hkv * shape.d * 2 * 2
    layout = wl.layout_pages(3, lens, shape.P, shared_prefix=16384, width=8192)
    distinct = len(set(np.concatenate(layout.pages).tolist())) * shape.P * shape.Hkv * shape.d * 2 * 2
    lines, fetch_b, write_b, avg_ns = _decode_profile_lines(
        trace_dir, pmc_dir, "shared", alg,
        "decode_split_kernel<128, bf16> -- Llama-3.1-70B-shaped decode, 128 sequences on a shared "
        "16384-token prefix",
        "64 query / 8 KV heads, head_dim 128, bf16 pages of 16 tokens, fixed 2048-token splits; 128 sequences = "
        "one 16384-token prefix held once in 1024 refcounted pages + private suffixes of 256-4096 tokens; "
        f"block tables 8192 wide (131072 keys); IA_KV_HINT_CACHED.  Logical KV bytes per launch {alg} (what the "
        f"128 sequences read); bytes of the distinct pages {distinct}.",
        "--shared-prefix-only", 3)
    lines += [
        "## Logical against DRAM bytes",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| logical KV bytes per launch | {alg:.4e} |",
        f"| distinct-page bytes | {distinct:.4e} |",
        f"| bytes the L2s fetch from the fabric per launch (FETCH_SIZE, calibrated) | {fetch_b:.4e} |",
        f"| fetched / distinct-page bytes | {fetch_b / distinct:.3f} |",
        f"| fetched / logical bytes | {fetch_b / alg:.3f} |",
        f"| logical rate | {alg / avg_ns:.1f} GB/s |",
        f"| DRAM-side rate (fetched bytes / kernel time) | {fetch_b / avg_ns:.1f} GB/s = "
        f"{fetch_b / avg_ns / HBM_PEAK_GBS:.4f} of peak |",
        "",
        "FETCH_SIZE counts what the L2s read from the data fabric, which the 256 MB last-level cache (MALL) "
        "serves before HBM, so the fetched bytes bound the HBM bytes from above.  Each of the 8 XCDs has its "
        "own L2, and sequences at different points of the prefix evict each other's lines from the 4 MB L2s, "
        "so a shared page is fetched more than once per launch; the 64 MiB prefix itself fits the MALL.  The "
        "logical rate (what the 128 sequences read) is above the HBM peak because most of the shared bytes "
        "come from the caches.",
        "",
    ]
    with open(SHARED_PREFIX_PROFILE_MD, "w") as f:
        f.write("\n".join(lines))
    print(SHARED_PREFIX_PROFILE_MD)


SPREAD_PROFILE_MD = os.path.join(ROOT, "profiles", "decode_spread_kernels_llama3-8b_b1.md")
MIXED_PROFILE_MD = os.path.join(ROOT, "profiles", "prefill_split_grid_qwen3-235b_mixed.md")


def summarize_spread_profile(trace_dir):
    """Writes the kernel-trace summary of one batch-1 decode call on the spread kernels."""
    stats = _csv_rows(os.path.join(trace_dir, "**", "*kernel_stats.csv"))
    names = ["decode_score_kernel<128, false>", "decode_weight_kernel<128, false>",
             "decode_value_kernel<128, false, 1>", "decode_merge_kernel<128, false>"]
    rows = [r for n in names for r in stats if n in r["Name"]]
    lens = wl.uniform_lens(SEED, 256, 512, 8192)[:1]
    alg = int(sum(lens)) * 8 * 128 * 2 * 2
    total = sum(float(r["AverageNs"]) for r in rows)
    cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o spread -- "
           "python3 bench.py --decode-only --no-cpu-baseline --batch 1 --steps 20 --warmup 5")
    lines = [
        "# decode spread kernels -- Llama-3-8B-shaped decode, batch 1",
        "",
        f"32 query / 8 KV heads, head_dim 128, bf16 pages of 16 tokens, fixed 2048-token splits, one sequence of "
        f"{int(sum(lens))} keys (the first of the batch-256 workload): 4 splits x 8 KV heads = 32 split units, "
        f"which IA_DECODE_AUTO runs on the spread kernels; algorithmic KV bytes per call {alg}.",
        "",
        "## Kernel trace (rocprofv3 --kernel-trace --stats)",
        "",
        f"    {cmd}",
        "",
        "| kernel | calls | average ns | min ns | max ns |",
        "|---|---|---|---|---|",
    ]
    for r in rows:
        lines.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")
    lines += [
        "",
        f"Sum of the four kernels' average durations: {total / 1e3:.1f} us per decode call "
        f"({alg / total:.1f} GB/s of algorithmic KV bytes, {alg / total / HBM_PEAK_GBS:.4f} of the 8 TB/s peak). "
        "Each kernel is about one round trip to memory plus its launch; the value kernel holds two round trips "
        "(block-table entries, then the copies) and the 32-step chain of one split.",
        "",
    ]
    with open(SPREAD_PROFILE_MD, "w") as f:
        f.write("\n".join(lines))
    print(SPREAD_PROFILE_MD)


def summarize_mixed_profile(trace_dir):
    """Writes the kernel-trace summary of the Qwen3-235B mixed prefill call under the automatic grid
    (prefill_kernel with one workgroup per split for the decode rows, then prefill_merge_kernel)
    and under in-workgroup folds (prefill_kernel alone), from bench.py --mixed-only."""
    trace = sorted(_csv_rows(os.path.join(trace_dir, "**", "*kernel_trace.csv")), key=lambda r: int(r["Start_Timestamp"]))
    dur = lambda r: int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    split, merge, fold = [], [], []
    for i, r in enumerate(trace):
        if "prefill_kernel<" not in r["Kernel_Name"]:
            continue
        nxt = trace[i + 1]["Kernel_Name"] if i + 1 < len(trace) else ""
        if "prefill_merge_kernel<" in nxt:
            split.append(dur(r))
            merge.append(dur(trace[i + 1]))
        else:
            fold.append(dur(r))
    name = next((r["Kernel_Name"] for r in trace if "prefill_kernel<" in r["Kernel_Name"]), "prefill_kernel")
    mname = next((r["Kernel_Name"] for r in trace if "prefill_merge_kernel<" in r["Kernel_Name"]), "prefill_merge_kernel")
    stat = lambda v: (f"{len(v)} | {sum(v) / len(v):.0f} | {min(v)} | {max(v)}") if v else "0 | - | - | -"
    cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o mixed -- "
           "python3 bench.py --mixed-only --steps 20 --warmup 5")
    lines = [
        "# prefill split grid -- Qwen3-235B-shaped mixed prefill call",
        "",
        "64 query / 4 KV heads, head_dim 128, bf16 pages of 16 tokens, fixed 2048-token splits; one prefill call of "
        "16 one-row decode queries at 32768 keys and 4 fresh 512-token prompts, first under the automatic prefill "
        "grid (each decode row's sequence runs one workgroup per (row block, KV head, split), then the merge "
        "kernel folds the split states), then under in-workgroup folds (one workgroup per (row block, KV head) "
        "walks all 512 tiles). Both give the same bits.",
        "",
        "## Kernel trace (rocprofv3 --kernel-trace)",
        "",
        f"    {cmd}",
        "",
        "| launch | kernel | dispatches | average ns | min ns | max ns |",
        "|---|---|---|---|---|---|",
        f"| automatic grid | {name} | {stat(split)} |",
        f"| automatic grid | {mname} | {stat(merge)} |",
        f"| in-workgroup folds | {name} | {stat(fold)} |",
        "",
    ]
    if split and fold:
        a = (sum(split) + sum(merge)) / len(split)
        f = sum(fold) / len(fold)
        lines += [f"Per call: {a / 1e3:.1f} us under the automatic grid (attention and merge kernels) against "
                  f"{f / 1e3:.1f} us under in-workgroup folds ({f / a:.2f}x).", ""]
    with open(MIXED_PROFILE_MD, "w") as fh:
        fh.write("\n".join(lines))
    print(MIXED_PROFILE_MD)


PREFILL_KERNEL = "prefill_kernel<128, false, 2>"
PREFILL_SQ = ["SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
              "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAVES"]
# A second pass: issue, co-execution and waits (the SQ block takes at most 8 counters a run).
PREFILL_SQ2 = ["SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_COEXEC_CYCLES",
               "SQ_INSTS_VALU_TRANS_F32", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_LDS"]


LAYER_SHAPES = [("qkv_proj", 8192, 6144, 4096), ("down_proj", 8192, 4096, 14336), ("qkv_proj", 256, 6144, 4096),
                ("down_proj", 256, 4096, 14336)]


def summarize_layer_profile(trace_dir, layer_json):
    """Writes the layer-operator profile summary: per-shape median kernel time from a kernel trace of
    `bench.py --layer-only`, beside the vendor library's rate from that run's own JSON line."""
    trace = _csv_rows(os.path.join(trace_dir, "**", "*kernel_trace.csv"))
    with open(layer_json) as f:
        lo = json.loads([ln for ln in f.read().splitlines() if ln.startswith("{")][-1])["layer_ops"]

    def wgs(r):
        return int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])

    def tile_of(name):
        m = re.search(r"TileILi(\d+)ELi(\d+)ELi\d+ELi\d+ELi(\d+)E", name) or re.search(
            r"Tile<(\d+), (\d+), \d+, \d+, (\d+)>", name)
        return f"{m.group(1)}x{m.group(2)}, K step {m.group(3)}, 2 slots" if m else name

    cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o layer -- "
           "python3 bench.py --layer-only --steps 10 --warmup 10")
    lines = [
        "# gemm_kernel / rmsnorm_kernel -- Llama-3-8B / Qwen3-8B layer shapes (batch-invariant layer operators)",
        "",
        "C = A W^T with bf16 A [M][K] and W [N][K], fp32 accumulation, bf16 C; one MFMA chain over k per output. "
        "The 256 x 256 tile runs when it gives at least one workgroup per compute unit, else the 64 x 64 tile, "
        "with K steps of 128 when K allows and its tiles fit one round of the compute units (same bits every "
        "way).  RMSNorm: 8192 rows of 4096.",
        "",
        "## Kernel trace (rocprofv3 --kernel-trace)",
        "",
        f"    {cmd}",
        "",
        "Median over the dispatches of each shape (warmup included; the median is past the clock ramp).",
        "",
        "| kernel | shape | workgroups | dispatches | median ns | TFLOP/s (median) | fraction of 2.5 PFLOP/s |",
        "|---|---|---|---|---|---|---|",
    ]
    vendor = []
    for name, M, N, K in LAYER_SHAPES:
        big = (N // 256) * ((M + 255) // 256)
        ngroups = big if big >= 256 else (N // 64) * ((M + 63) // 64)
        rows = [r for r in trace if "gemm_kernel" in r["Kernel_Name"] and wgs(r) == ngroups]
        d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]
        med = float(np.median(d))
        tf = 2.0 * M * N * K / med / 1e3
        lines.append(f"| gemm_kernel<{tile_of(rows[0]['Kernel_Name'])}> | {name} M={M} (N={N}, K={K}) | {ngroups} | "
                     f"{len(d)} | {med:.0f} | {tf:.1f} | {tf / BF16_PEAK_TFLOPS:.4f} |")
        vendor.append(f"{lo['gemm'][f'{name}_M{M}']['torch_tflops'] / 1e3:.2f} PFLOP/s ({name} M={M})")
    rn = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace if "rmsnorm_kernel" in r["Kernel_Name"]]
    med = float(np.median(rn))
    gbs = 2 * 8192 * 4096 * 2 / med
    lines += [
        "",
        "| kernel | shape | dispatches | median ns | GB/s (read x + write y) | fraction of 8 TB/s |",
        "|---|---|---|---|---|---|",
        f"| rmsnorm_kernel | 8192 x 4096 | {len(rn)} | {med:.0f} | {gbs:.1f} | {gbs / HBM_PEAK_GBS:.4f} |",
        "",
        "The vendor library (torch.matmul on hipBLASLt) on the same shapes, timed by `bench.py --layer-only` in "
        "the same traced run: " + ", ".join(vendor) + f".  Row 0 computed alone equals row 0 inside the "
        f"8192-row batch: ours {lo['row0_alone_equals_in_batch']['ours']}, the vendor library's "
        f"{lo['row0_alone_equals_in_batch']['torch']}.",
        "",
    ]
    out = os.path.join(ROOT, "profiles", "gemm_rmsnorm_llama3-8b-layer.md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(out)


PREFILL_PROFILE_STEPS = 10


def summarize_prefill_profile(trace_dir, pmc_dir):
    """Writes the prefill profile summary: kernel-trace stats, executed MFMA work from SQ counters and
    calibrated FETCH/WRITE bytes."""
    stats = _csv_rows(os.path.join(trace_dir, "**", "*kernel_stats.csv"))
    rows = [r for r in stats if PREFILL_KERNEL in r["Name"]]
    # The first dispatches run while the clock ramps up: the achieved rate is taken over the timed
    # calls, the last PREFILL_PROFILE_STEPS dispatches of the traced run.
    trace = _csv_rows(os.path.join(trace_dir, "**", "*kernel_trace.csv"))
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace if PREFILL_KERNEL in r["Kernel_Name"]]
    timed = durs[-PREFILL_PROFILE_STEPS:]
    avg_ns = float(np.mean(timed))
    shape = wl.QWEN3_8B
    lens = [4096] * 8
    flops = 4.0 * shape.d * shape.Hq * sum(n * (n + 1) / 2 for n in lens)
    kv_unique = sum(lens) * shape.Hkv * shape.d * 2 * 2
    pm = {c: _pmc_mean(pmc_dir, "prefill", c, PREFILL_KERNEL) for c in PREFILL_SQ + PREFILL_SQ2}
    fetch_kib, nf = _pmc_mean(pmc_dir, "prefill", "FETCH_SIZE", PREFILL_KERNEL)
    write_kib, nw = _pmc_mean(pmc_dir, "prefill", "WRITE_SIZE", PREFILL_KERNEL)
    copy_fetch, _ = _pmc_mean(pmc_dir, "copy", "FETCH_SIZE", "__amd_rocclr_copyBuffer")
    copy_write, _ = _pmc_mean(pmc_dir, "copy", "WRITE_SIZE", "__amd_rocclr_copyBuffer")
    f_scale = COPY_PROBE_BYTES / (copy_fetch * 1024)
    w_scale = COPY_PROBE_BYTES / (copy_write * 1024)
    mfma_flops = pm["SQ_INSTS_MFMA"][0] * MFMA_FLOPS
    cmd_trace = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o prefill -- "
                 f"python3 bench.py --prefill-only --steps {PREFILL_PROFILE_STEPS} --warmup 30")
    cmd_sq = ("rocprofv3 --pmc " + " ".join(PREFILL_SQ) + " --output-format csv -d <out> -o pmc -- "
              "python3 bench.py --prefill-only --steps 3 --warmup 1")
    cmd_sq2 = ("rocprofv3 --pmc " + " ".join(PREFILL_SQ2) + " --output-format csv -d <out> -o pmc -- "
               "python3 bench.py --prefill-only --steps 3 --warmup 1")
    cmd_pmc = ("rocprofv3 --pmc {C} --output-format csv -d <out> -o pmc -- "
               "python3 bench.py --prefill-only --steps 3 --warmup 1")
    cmd_copy = "rocprofv3 --pmc {C} --output-format csv -d <out> -o pmc -- python3 bench.py --copy-probe --steps 3"
    tf = flops / avg_ns / 1e3
    ws_rows = sum(max(0, n - shape.S) for n in lens) * shape.Hq  # rows that see two splits
    ws_bytes = ws_rows * (shape.d + 2) * 4
    lines = [
        "# prefill_kernel<128, bf16, 2 row blocks per wave> -- Qwen3-8B-shaped whole prefill, 8 prompts x 4096 tokens, causal",
        "",
        "32 query / 8 KV heads, head_dim 128, bf16 pages of 16 tokens, fixed 2048-token splits; algorithmic "
        f"flops per launch {flops:.6e} (4 x d x Hq x sum over rows of the p + 1 visible keys).",
        "",
        "## Kernel trace (rocprofv3 --kernel-trace --stats)",
        "",
        f"    {cmd_trace}",
        "",
        "| kernel | calls | average ns | min ns | max ns |",
        "|---|---|---|---|---|",
    ]
    for r in rows:
        lines.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")
    lines += [
        "",
        f"Timed calls (the last {len(timed)} dispatches, after 30 warmup calls during which the clock ramps up): "
        f"mean {avg_ns:.0f} ns, min {min(timed)} ns, max {max(timed)} ns.",
        "",
        f"Achieved over the timed calls: {tf:.1f} TFLOP/s = {tf / BF16_PEAK_TFLOPS:.4f} of the 2.5 PFLOP/s dense "
        "bf16 peak.",
        "",
        "## MFMA work and issue (rocprofv3 --pmc, SQ counters, one run)",
        "",
        f"    {cmd_sq}",
        "",
        "| quantity | value |",
        "|---|---|",
    ]
    for c in PREFILL_SQ:
        lines.append(f"| {c} per dispatch (mean of {pm[c][1]}) | {pm[c][0]:.4e} |")
    lines += [
        f"| executed MFMA flops (SQ_INSTS_MFMA x {MFMA_FLOPS}) | {mfma_flops:.4e} |",
        f"| executed / algorithmic flops | {mfma_flops / flops:.4f} |",
        f"| MFMA pipe busy (executed flops / (duration x peak)) | {mfma_flops / (avg_ns * 1e-9) / 2.5e15:.4f} |",
        f"| LDS bank-conflict cycles / LDS active cycles | "
        f"{pm['SQ_LDS_BANK_CONFLICT'][0] / pm['SQ_LDS_IDX_ACTIVE'][0]:.4f} |",
        "",
        "Executed over algorithmic flops is 1.5 plus masking waste: each weight is carried as a bf16 hi/lo "
        "pair, so the value product runs two MFMAs per k-step.",
        "",
        "Second pass (issue, co-execution and waits):",
        "",
        f"    {cmd_sq2}",
        "",
        "| quantity | value |",
        "|---|---|",
    ]
    for c in PREFILL_SQ2:
        lines.append(f"| {c} per dispatch (mean of {pm[c][1]}) | {pm[c][0]:.4e} |")
    coexec = pm["SQ_VALU_MFMA_COEXEC_CYCLES"][0] / pm["SQ_VALU_MFMA_BUSY_CYCLES"][0]
    lines += [
        f"| VALU-MFMA co-execution cycles / MFMA busy cycles | {coexec:.4f} |",
        f"| exp2 (SQ_INSTS_VALU_TRANS_F32) / MFMA instructions | "
        f"{pm['SQ_INSTS_VALU_TRANS_F32'][0] / pm['SQ_INSTS_MFMA'][0]:.4f} |",
        "",
        "## HBM traffic (rocprofv3 --pmc, one counter per run)",
        "",
        f"    {cmd_pmc.format(C='FETCH_SIZE')}",
        f"    {cmd_pmc.format(C='WRITE_SIZE')}",
        f"    {cmd_copy.format(C='FETCH_SIZE')}",
        f"    {cmd_copy.format(C='WRITE_SIZE')}",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| FETCH_SIZE per dispatch (KiB, mean of {nf}) | {fetch_kib:.1f} |",
        f"| WRITE_SIZE per dispatch (KiB, mean of {nw}) | {write_kib:.1f} |",
        f"| fetch / write scale (1 GiB device copy) | {f_scale:.4f} / {w_scale:.4f} |",
        f"| HBM bytes read per launch | {fetch_kib * 1024 * f_scale:.4e} |",
        f"| HBM bytes written per launch | {write_kib * 1024 * w_scale:.4e} |",
        f"| distinct K/V bytes (read at least once) | {kv_unique:.4e} |",
        f"| Q bytes read + O bytes written | {2 * sum(lens) * shape.Hq * shape.d * 2:.4e} |",
        f"| split-merge workspace bytes written, then read (rows past the first split) | {ws_bytes:.4e} |",
        "",
    ]
    os.makedirs(os.path.dirname(PREFILL_PROFILE_MD), exist_ok=True)
    with open(PREFILL_PROFILE_MD, "w") as f:
        f.write("\n".join(lines))
    print(PREFILL_PROFILE_MD)


def make_ctx(shape, by_count=False, fp8=False, decode_kernel=None, kv_cache_hint=None, prefill_grid=None):
    return ia.Context(ia.make_config(shape.Hq, shape.Hkv, shape.d, page_size=shape.P, split_tokens=shape.S,
                                     kv_dtype=ia.IA_KV_FP8_E4M3 if fp8 else ia.IA_KV_BF16,
                                     split_policy=ia.IA_SPLIT_BY_COUNT if by_count else ia.IA_SPLIT_FIXED,
                                     sm_scale=shape.scale,
                                     decode_kernel=ia.IA_DECODE_AUTO if decode_kernel is None else decode_kernel,
                                     kv_cache_hint=ia.IA_KV_HINT_AUTO if kv_cache_hint is None else kv_cache_hint,
                                     prefill_grid=ia.IA_PREFILL_AUTO if prefill_grid is None else prefill_grid))


class DecodeWorld:
    """A decode workload resident on the GPU: pages, tables, queries, new-token rows, slots."""

    def __init__(self, shape: wl.AttnShape, lens, fp8=False, shared_prefix=0, width=None, scales=None,
                 layout_seed=3, gpu_values=False, keep_host=False):
        """gpu_values: K/V/Q drawn on the GPU from a seeded torch generator (N(0,1) rounded to bf16), for
        the large timing-only worlds; otherwise from synth.workloads on the host (the tests' values).
        keep_host: keep the host rows (bf16) so the oracle can scatter the same values."""
        self.shape = shape
        self.lens = [int(n) for n in lens]
        self.B = len(self.lens)
        self.fp8 = fp8
        self.seqs = wl.make_sequences(self.lens, shared_prefix=shared_prefix)
        self.layout = wl.layout_pages(layout_seed, self.lens, shape.P, shared_prefix=shared_prefix, width=width)
        self.ctx = make_ctx(shape, fp8=fp8)
        dt = torch.uint8 if fp8 else torch.bfloat16
        npg = self.layout.num_pages
        self.k = torch.zeros((npg, shape.Hkv, shape.d // 8, shape.P, 8), dtype=dt, device=DEV)
        self.v = torch.zeros((npg, shape.Hkv, shape.d, shape.P), dtype=dt, device=DEV)
        if fp8:
            ks, vs = scales if scales is not None else wl.fp8_scales(2, shape.Hkv, power_of_two=False)
            self.k_scale = torch.as_tensor(ks, device=DEV)
            self.v_scale = torch.as_tensor(vs, device=DEV)
        else:
            self.k_scale = self.v_scale = None
        t0 = time.time()
        qs, knew, vnew, slots = [], [], [], []
        self.host_rows = [] if keep_host else None
        n_shared = shared_prefix // shape.P
        gen = None
        if gpu_values:
            gen = torch.Generator(device=DEV)
            gen.manual_seed(SEED * 1000003 + layout_seed)
        for b, s in enumerate(self.seqs):
            # Shared prefix pages are written once (by the first sequence), as a prefix cache would.
            p0 = 0 if b == 0 else min(s.n, n_shared * shape.P)
            if gen is not None:
                kr = torch.randn((s.n - p0, shape.Hkv, shape.d), generator=gen, device=DEV).to(torch.bfloat16)
                vr = torch.randn((s.n - p0, shape.Hkv, shape.d), generator=gen, device=DEV).to(torch.bfloat16)
                qr = torch.randn((1, shape.Hq, shape.d), generator=gen, device=DEV).to(torch.bfloat16)
            else:
                kr = s.k(SEED, shape, p0, s.n)
                vr = s.v(SEED, shape, p0, s.n)
                qr = s.q(SEED, shape, s.n - 1, s.n)
            if keep_host:
                self.host_rows.append((p0, kr.cpu(), vr.cpu()))
            sl = torch.as_tensor(self.layout.slots(b, p0, s.n, shape.P), device=DEV)
            ia.ia_kv_append(self.ctx, kr.to(DEV), vr.to(DEV), sl, self.k, self.v, self.k_scale, self.v_scale)
            qs.append(qr.to(DEV))
            knew.append(kr[-1:].to(DEV))
            vnew.append(vr[-1:].to(DEV))
            slots.append(self.layout.slots(b, s.n - 1, s.n, shape.P))
        torch.cuda.synchronize()
        log(f"  filled {self.B} sequences ({sum(self.lens)} tokens) in {time.time() - t0:.1f}s")
        self.q = torch.cat(qs).to(DEV)
        self.k_new = torch.cat(knew).to(DEV)
        self.v_new = torch.cat(vnew).to(DEV)
        self.slots = torch.as_tensor(np.concatenate(slots), device=DEV)
        self.bt = torch.as_tensor(self.layout.block_table, device=DEV)
        self.seq_lens = torch.as_tensor(np.array(self.lens, np.int32), device=DEV)
        self.distinct_pages = len(set(np.concatenate(self.layout.pages).tolist()))

    def kv_bytes(self, idx=None) -> int:
        """Algorithmic (logical) KV bytes: every sequence reads its whole context once per KV head."""
        lens = self.lens if idx is None else [self.lens[i] for i in idx]
        return int(sum(lens)) * self.shape.Hkv * self.shape.d * 2 * (1 if self.fp8 else 2)


class DecodeRunner:
    """One batch (a subset of the world's sequences) ready to step."""

    def __init__(self, world: DecodeWorld, idx, ctx=None):
        self.w = world
        idx = list(idx)
        self.idx = idx
        self.B = len(idx)
        self.ctx = world.ctx if ctx is None else ctx
        ii = torch.as_tensor(idx, device=DEV)
        self.q = world.q[ii].contiguous()
        self.bt = world.bt[ii].contiguous()
        self.sl = world.seq_lens[ii].contiguous()
        self.k_new = world.k_new[ii].contiguous()
        self.v_new = world.v_new[ii].contiguous()
        self.slots = world.slots[ii].contiguous()
        self.max_len = max(world.lens[i] for i in idx)
        self.out = torch.empty((self.B, world.shape.Hq, world.shape.d), dtype=torch.bfloat16, device=DEV)
        nb = ia.ia_decode_workspace_bytes(self.ctx, self.B, self.max_len)
        self.ws = torch.empty(nb, dtype=torch.uint8, device=DEV)

    def append(self, stream):
        ia.ia_kv_append(self.ctx, self.k_new, self.v_new, self.slots, self.w.k, self.w.v, self.w.k_scale,
                        self.w.v_scale, stream=stream)

    def decode(self, stream):
        ia.ia_paged_attn_decode(self.ctx, self.q, self.w.k, self.w.v, self.bt, self.sl, self.max_len, self.out,
                                self.ws, self.w.k_scale, self.w.v_scale, stream=stream)


FLUSH_BYTES = 512 << 20
_flush_buf = None
_flush_out = None


def flush_caches(stream):
    """Reads a 512 MiB buffer: the L2s and the 256 MB MALL then hold none of the workload's data.
    (A read, not a write: written lines would be written back to HBM during the timed call.)"""
    global _flush_buf, _flush_out
    if _flush_buf is None:
        _flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=DEV)
    with torch.cuda.stream(stream):
        _flush_out = _flush_buf.sum()


def time_steps(runner: DecodeRunner, steps: int, warmup: int, with_append=True, flush=False):
    """Times `steps` steps.  Returns (ms per step over the whole timed region, mean ms of the decode
    call alone).  All work goes to torch's current stream, which the events are recorded on.
    flush: a 512 MiB read before each decode call (outside its events; the step time then
    includes it), so the call reads its K/V from HBM rather than from the caches."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        if with_append:
            runner.append(stream)
        runner.decode(stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for e1, e2 in ev:
        if with_append:
            runner.append(stream)
        if flush:
            flush_caches(stream)
        e1.record(stream)
        runner.decode(stream)
        e2.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / steps
    calls = [e1.elapsed_time(e2) for e1, e2 in ev]
    time_steps.last_calls = calls  # per-call decode times of the last measurement (for percentiles)
    dec_ms = float(np.mean(calls))
    return step_ms, dec_ms


def invariance_pairs(world: DecodeWorld, ctx, probes):
    """Bitwise comparisons of output rows across batch compositions: the full batch against each
    probe alone, the first 8, the first 64 and the reversed batch.  Returns (equal, compared)."""
    B = world.B
    full = DecodeRunner(world, range(B), ctx)
    full.decode(None)
    ref = full.out.clone()
    eq = tot = 0

    def cmp(idx):
        nonlocal eq, tot
        r = DecodeRunner(world, idx, ctx)
        r.decode(None)
        a = r.out.view(torch.int16).cpu().numpy().reshape(len(idx), -1)
        b = ref[torch.as_tensor(idx, device=DEV)].view(torch.int16).cpu().numpy().reshape(len(idx), -1)
        eq += int((a == b).all(axis=1).sum())
        tot += len(idx)

    for p in probes:
        cmp([p])
    for sub in (list(range(8)), list(range(64))):
        cmp(sub)
    cmp(list(reversed(range(B))))
    return eq, tot


def _row_bits(t):
    return t.view(torch.int16).cpu().numpy().reshape(t.shape[0], -1)


def _equal_rows(a, b):
    return int((_row_bits(a) == _row_bits(b)).all(axis=1).sum()), int(a.shape[0])


def _prefill_world(shape, lens, layout_seed):
    """Pages, queries and tables of whole prompts (every position's K/V appended)."""
    seqs = wl.make_sequences(lens, first_sid=2000)
    layout = wl.layout_pages(layout_seed, lens, shape.P)
    ctx = make_ctx(shape)
    k = torch.zeros((layout.num_pages, shape.Hkv, shape.d // 8, shape.P, 8), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((layout.num_pages, shape.Hkv, shape.d, shape.P), dtype=torch.bfloat16, device=DEV)
    for b, s in enumerate(seqs):
        sl = torch.as_tensor(layout.slots(b, 0, s.n, shape.P), device=DEV)
        ia.ia_kv_append(ctx, s.k(SEED, shape).to(DEV), s.v(SEED, shape).to(DEV), sl, k, v)
    return seqs, layout, ctx, k, v


def prefill_workspace(ctx, B, total_q, max_q_len, max_seq_len):
    """The prefill workspace for a launch (None when its rows see one split only)."""
    n = ia.ia_prefill_workspace_bytes(ctx, int(B), int(total_q), int(max_q_len), int(max_seq_len))
    return torch.empty(n, dtype=torch.uint8, device=DEV) if n else None


def _prefill_rows(shape, seqs, layout, ctx, k, v, p0, p1):
    """Rows p0 .. p1 - 1 of every prompt in one prefill call (key length p1)."""
    q = torch.cat([s.q(SEED, shape, p0, p1) for s in seqs]).to(DEV)
    B = len(seqs)
    cu = torch.as_tensor(np.arange(0, B * (p1 - p0) + 1, p1 - p0, dtype=np.int32), device=DEV)
    sl = torch.as_tensor(np.full(B, p1, np.int32), device=DEV)
    bt = torch.as_tensor(layout.block_table, device=DEV)
    out = torch.empty_like(q)
    ia.ia_paged_attn_prefill(ctx, q, cu, sl, k, v, bt, p1 - p0, p1, out,
                             workspace=prefill_workspace(ctx, B, q.shape[0], p1 - p0, p1))
    return out.view(B, p1 - p0, shape.Hq, shape.d)


def invariance_variations(lens):
    """Bitwise comparisons for the execution variations other than batch composition: the
    Llama-3-8B decode rows of 8 sequences on a second random page placement and with a 16x wider
    block table, decode against prefill at 16 positions of each, and the Qwen3-8B prefill of 2
    prompts of 4096 tokens whole against chunks of 64 / 256 / 1024 and against its second half
    served from pages written by an earlier call (a cached 2048-token prefix).  A pair is one
    output row (all query heads).  Returns {variation: (equal, compared)}."""
    res = {}
    shape = wl.LLAMA3_8B
    lens8 = [int(x) for x in lens[:8]]
    w1 = DecodeWorld(shape, lens8)
    w2 = DecodeWorld(shape, lens8, layout_seed=7)
    wide = DecodeWorld(shape, lens8, width=16 * (max(lens8) // shape.P + 1))
    r1, r2, r3 = DecodeRunner(w1, range(8)), DecodeRunner(w2, range(8)), DecodeRunner(wide, range(8))
    for r in (r1, r2, r3):
        r.decode(None)
    res["decode_page_placement"] = _equal_rows(r2.out, r1.out)
    res["decode_table_width"] = _equal_rows(r3.out, r1.out)
    # decode at n' = n - j against the prefill rows of the last 16 positions (keys past n' exist
    # in the pages but are causally masked)
    eq = tot = 0
    q16 = torch.cat([w1.seqs[b].q(SEED, shape, lens8[b] - 16, lens8[b]) for b in range(8)]).to(DEV)
    cu = torch.as_tensor(np.arange(0, 8 * 16 + 1, 16, dtype=np.int32), device=DEV)
    sl = torch.as_tensor(np.array(lens8, np.int32), device=DEV)
    pre = torch.empty((8 * 16, shape.Hq, shape.d), dtype=torch.bfloat16, device=DEV)
    ia.ia_paged_attn_prefill(w1.ctx, q16, cu, sl, w1.k, w1.v, w1.bt, 16, max(lens8), pre,
                             workspace=prefill_workspace(w1.ctx, 8, q16.shape[0], 16, max(lens8)))
    pre = pre.view(8, 16, shape.Hq, shape.d)
    ws = torch.empty(ia.ia_decode_workspace_bytes(w1.ctx, 8, max(lens8)), dtype=torch.uint8, device=DEV)
    for j in range(16):
        nj = [n - 16 + j + 1 for n in lens8]
        qd = torch.stack([q16[b * 16 + j] for b in range(8)])
        out = torch.empty((8, shape.Hq, shape.d), dtype=torch.bfloat16, device=DEV)
        ia.ia_paged_attn_decode(w1.ctx, qd, w1.k, w1.v, w1.bt, torch.as_tensor(np.array(nj, np.int32), device=DEV),
                                max(lens8), out, ws)
        e, t = _equal_rows(out, pre[:, j])
        eq, tot = eq + e, tot + t
    res["decode_vs_prefill"] = (eq, tot)
    del w1, w2, wide, r1, r2, r3
    torch.cuda.empty_cache()
    shape = wl.QWEN3_8B
    n = 4096
    seqs, layout, ctx, k, v = _prefill_world(shape, [n, n], 11)
    whole = _prefill_rows(shape, seqs, layout, ctx, k, v, 0, n)
    for budget in (64, 256, 1024):
        parts = [_prefill_rows(shape, seqs, layout, ctx, k, v, c0, min(n, c0 + budget)) for c0 in range(0, n, budget)]
        chunked = torch.cat(parts, dim=1)
        res[f"prefill_chunks_{budget}"] = _equal_rows(chunked.reshape(-1, shape.Hq, shape.d),
                                                     whole.reshape(-1, shape.Hq, shape.d))
    half = _prefill_rows(shape, seqs, layout, ctx, k, v, n // 2, n)
    res["prefill_cached_prefix_2048"] = _equal_rows(half.reshape(-1, shape.Hq, shape.d),
                                                     whole[:, n // 2:].reshape(-1, shape.Hq, shape.d))
    return res


def copy_gbs(nbytes=COPY_PROBE_BYTES, reps=10):
    """A plain device copy (torch's copy kernel) of nbytes: read + write bytes / time."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=DEV).normal_()
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": round(ms, 4), "gbs": round(2 * nbytes / ms / 1e6, 1)}


def read_gbs(nbytes=4 * COPY_PROBE_BYTES, reps=10):
    """A plain device read (torch's sum over 4 GiB of fp32): bytes read / time."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=DEV)
    for _ in range(2):
        src.sum()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        src.sum()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src
    torch.cuda.empty_cache()
    return {"bytes_read": nbytes, "ms": round(ms, 4), "gbs": round(nbytes / ms / 1e6, 1)}


def prefill_tflops(steps: int, warmup: int):
    """Whole prefill of 8 prompts x 4096 tokens (Qwen3-8B shape); flops = 4 d Hq sum_rows (p+1)."""
    shape = wl.QWEN3_8B
    lens = [4096] * 8
    seqs = wl.make_sequences(lens, first_sid=1000)
    layout = wl.layout_pages(5, lens, shape.P)
    ctx = make_ctx(shape)
    k = torch.zeros((layout.num_pages, shape.Hkv, shape.d // 8, shape.P, 8), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((layout.num_pages, shape.Hkv, shape.d, shape.P), dtype=torch.bfloat16, device=DEV)
    qs = []
    for b, s in enumerate(seqs):
        sl = torch.as_tensor(layout.slots(b, 0, s.n, shape.P), device=DEV)
        ia.ia_kv_append(ctx, s.k(SEED, shape).to(DEV), s.v(SEED, shape).to(DEV), sl, k, v)
        qs.append(s.q(SEED, shape, 0, s.n))
    q = torch.cat(qs).to(DEV)
    cu = torch.as_tensor(np.arange(0, 8 * 4096 + 1, 4096, dtype=np.int32), device=DEV)
    sl = torch.as_tensor(np.array(lens, np.int32), device=DEV)
    bt = torch.as_tensor(layout.block_table, device=DEV)
    out = torch.empty_like(q)
    ws = prefill_workspace(ctx, 8, q.shape[0], 4096, 4096)
    stream = torch.cuda.current_stream()

    def run():
        ia.ia_paged_attn_prefill(ctx, q, cu, sl, k, v, bt, 4096, 4096, out, workspace=ws, stream=stream)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 4.0 * shape.d * shape.Hq * sum(n * (n + 1) / 2 for n in lens)
    return {"workload": "qwen3-8b-shaped whole prefill, 8 x 4096 tokens, causal", "ms": round(ms, 4),
            "tflops": round(flops / ms / 1e9, 1), "frac_of_bf16_peak": round(flops / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
            "algorithmic_flops": flops}


def layer_ops(steps: int, warmup: int):
    """The batch-invariant layer operators against torch's (vendor library) kernels on Llama-3-8B /
    Qwen3-8B layer shapes: the fixed-tile GEMM at a prefill chunk (M = 8192) and a decode batch
    (M = 256), RMSNorm at hidden 4096; plus whether torch's matmul keeps a row's bits when the
    batch changes."""
    from synth import layer_inputs as li

    def timed(f):
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    out = {"gemm": {}}
    shapes = {"qkv_proj": (6144, 4096), "down_proj": (4096, 14336)}
    for M in (8192, 256):
        for name, (N, K) in shapes.items():
            a = li.activations(SEED, 0, M, K).to(DEV)
            w = li.gemm_weight(SEED, N, K).to(DEV)
            c = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
            ms = timed(lambda: ia.ia_gemm_bf16(a, w, c))
            ms_t = timed(lambda: torch.matmul(a, w.t()))
            fl = 2.0 * M * N * K
            key = f"{name}_M{M}"
            out["gemm"][key] = {"M": M, "N": N, "K": K, "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                                "frac_of_bf16_peak": round(fl / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
                                "torch_ms": round(ms_t, 4), "torch_tflops": round(fl / ms_t / 1e9, 1),
                                "time_vs_torch": round(ms / ms_t, 3)}
            log(f"gemm {key}: {out['gemm'][key]}")
    # Row 0 alone vs inside the 8192-row batch: ours by construction, torch's as it happens.
    N, K = shapes["qkv_proj"]
    a = li.activations(SEED, 0, 8192, K).to(DEV)
    w = li.gemm_weight(SEED, N, K).to(DEV)
    c_full = torch.empty((8192, N), dtype=torch.bfloat16, device=DEV)
    c_one = torch.empty((1, N), dtype=torch.bfloat16, device=DEV)
    ia.ia_gemm_bf16(a, w, c_full)
    ia.ia_gemm_bf16(a[:1].contiguous(), w, c_one)
    t_full = torch.matmul(a, w.t())
    t_one = torch.matmul(a[:1].contiguous(), w.t())
    torch.cuda.synchronize()
    out["row0_alone_equals_in_batch"] = {"ours": bool(torch.equal(c_full[:1].view(torch.int16), c_one.view(torch.int16))),
                                         "torch": bool(torch.equal(t_full[:1].view(torch.int16), t_one.view(torch.int16)))}
    x = li.activations(SEED, 0, 8192, 4096).to(DEV)
    g = li.norm_weight(SEED, 4096).to(DEV)
    y = torch.empty_like(x)
    ms = timed(lambda: ia.ia_rmsnorm(x, g, 1e-5, y))
    out["rmsnorm"] = {"M": 8192, "H": 4096, "ms": round(ms, 4), "gbs": round(2 * x.numel() * 2 / ms / 1e6, 1),
                      "frac_of_hbm_peak": round(2 * x.numel() * 2 / ms / 1e6 / HBM_PEAK_GBS, 4)}
    log(f"rmsnorm: {out['rmsnorm']}; row 0 alone = in batch: {out['row0_alone_equals_in_batch']}")
    return out


def _oracle_decode_rate(shape, lens, rows_of, threads, layout_seed=9, repeat_to_s=0.0):
    """Times the fp64 oracle on the decode rows of sequences with the given lengths: host pools laid
    out by the oracle's own scatter of the rows rows_of(b) -> (K bf16, V bf16, Q bf16 of the last
    position).  Returns (seconds per pass, passes, KV bytes per pass, fp64 flops per pass)."""
    from oracle import oracle
    oracle.build(force=False)
    lens = [int(n) for n in lens]
    layout = wl.layout_pages(layout_seed, lens, shape.P)
    kshape, vshape = oracle.kv_cache_shapes(layout.num_pages, shape.Hkv, shape.d, shape.P)
    kc, vc = np.zeros(kshape, np.uint16), np.zeros(vshape, np.uint16)
    qs = []
    for b in range(len(lens)):
        k, v, q = rows_of(b)
        oracle.kv_append(k.view(torch.int16).numpy().view(np.uint16), v.view(torch.int16).numpy().view(np.uint16),
                         layout.slots(b, 0, lens[b], shape.P), kc, vc, Hkv=shape.Hkv, d=shape.d, P=shape.P)
        qs.append(q)
    q = torch.cat(qs).view(torch.int16).numpy().view(np.uint16)
    cu = np.arange(len(lens) + 1, dtype=np.int32)

    def once():
        oracle.paged_attention(q, cu, np.array(lens, np.int32), kc, vc, layout.block_table, Hq=shape.Hq,
                               Hkv=shape.Hkv, d=shape.d, P=shape.P, scale=shape.scale, nthreads=threads)

    t0 = time.perf_counter()
    once()
    dt = time.perf_counter() - t0
    passes = 1
    if repeat_to_s > dt:
        reps = min(200, int(math.ceil(repeat_to_s / max(dt, 1e-3))))
        t0 = time.perf_counter()
        for _ in range(reps):
            once()
        dt = (time.perf_counter() - t0) / reps
        passes = reps + 1
    kvb = int(sum(lens)) * shape.Hkv * shape.d * 2 * 2
    flops = 4.0 * shape.d * shape.Hq * sum(lens)  # q.k and p.v per key and query head
    return dt, passes, kvb, flops


def cpu_baseline(world: DecodeWorld):
    """The fp64 oracle, as it stands, timed on the host cores on the headline workload itself: the
    whole batch-256 decode (every sequence's decode row, all query heads) once on all host threads,
    plus single-thread figures for the tiny decode and for the first 8 sequences.  Its inputs are
    the same bf16 values the GPU saw, laid out by the oracle's own scatter."""
    from oracle import oracle
    threads = oracle.max_threads()
    shape = world.shape

    def rows_of(b):
        p0, k, v = world.host_rows[b]
        assert p0 == 0
        return k, v, world.q[b:b + 1].cpu()

    dt, passes, kvb, fl = _oracle_decode_rate(shape, world.lens, rows_of, threads)
    out = {"value": round(kvb / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"the whole batch-256 headline workload ({sum(world.lens)} tokens): every sequence's decode "
                     f"row over all {shape.Hq} query heads in fp64, one pass",
           "wall_s": round(dt, 3), "gflops_fp64": round(fl / dt / 1e9, 2), "cpu": cpu_model()}
    # Single thread: the first 8 sequences of the same workload, and the tiny decode (4 sequences,
    # 8 query / 2 kv heads, head_dim 64, contexts 17 / 100 / 211 / 300).
    dt8, p8, kv8, fl8 = _oracle_decode_rate(shape, world.lens[:8], rows_of, 1, repeat_to_s=3.0)
    tiny = wl.TINY
    tseqs = wl.make_sequences(list(wl.TINY_LENS))
    dtt, pt, kvt, flt = _oracle_decode_rate(
        tiny, list(wl.TINY_LENS), lambda b: (tseqs[b].k(SEED, tiny), tseqs[b].v(SEED, tiny),
                                             tseqs[b].q(SEED, tiny, tseqs[b].n - 1, tseqs[b].n)), 1,
        repeat_to_s=1.0)
    out["single_thread"] = {
        "llama3-8b-decode-B8": {"wall_s": round(dt8, 4), "passes": p8, "gbs": round(kv8 / dt8 / 1e9, 3),
                                "gflops_fp64": round(fl8 / dt8 / 1e9, 3)},
        "tiny-decode-B4": {"wall_s": round(dtt, 6), "passes": pt, "gbs": round(kvt / dtt / 1e9, 3),
                           "gflops_fp64": round(flt / dtt / 1e9, 3)}}
    return out


def stream_read_reference(nbytes=4 * COPY_PROBE_BYTES, reps=20):
    """The library's plain streaming-read kernel over nbytes: the achievable-HBM reference."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=DEV)
    sink = torch.empty(ia.ia_stream_read_sink_bytes() // 4, dtype=torch.int32, device=DEV)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        ia.ia_stream_read(src, sink, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        ia.ia_stream_read(src, sink, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src
    torch.cuda.empty_cache()
    return {"kernel": "stream_read_kernel (16-byte nontemporal loads, 8 in flight per thread, contiguous share per workgroup)", "bytes_read": nbytes,
            "ms": round(ms, 4), "gbs": round(nbytes / ms / 1e6, 1), "frac_of_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}


def kv_append_prefill_size(steps=20, warmup=5):
    """kv_append of a whole 8 x 4096-token prefill (Qwen3-8B shape: 32768 rows of 8 KV heads x 128,
    bf16 K and V) into a shuffled page pool: bytes read + written per second."""
    shape = wl.QWEN3_8B
    lens = [4096] * 8
    layout = wl.layout_pages(5, lens, shape.P)
    ctx = make_ctx(shape)
    k = torch.zeros((layout.num_pages, shape.Hkv, shape.d // 8, shape.P, 8), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((layout.num_pages, shape.Hkv, shape.d, shape.P), dtype=torch.bfloat16, device=DEV)
    T = sum(lens)
    g = torch.Generator(device=DEV)
    g.manual_seed(SEED + 17)
    kn = torch.randn((T, shape.Hkv, shape.d), generator=g, device=DEV).to(torch.bfloat16)
    vn = torch.randn((T, shape.Hkv, shape.d), generator=g, device=DEV).to(torch.bfloat16)
    slots = torch.as_tensor(np.concatenate([layout.slots(b, 0, n, shape.P) for b, n in enumerate(lens)]), device=DEV)
    stream = torch.cuda.current_stream()
    run = lambda: ia.ia_kv_append(ctx, kn, vn, slots, k, v, stream=stream)  # noqa: E731
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = 2 * (2 * T * shape.Hkv * shape.d * 2) + T * 8  # K and V read and written, plus the slots
    return {"rows": T, "ms": round(ms, 4), "gbs_read_plus_written": round(nbytes / ms / 1e6, 1),
            "frac_of_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}


def qwen235_mixed_call(w, steps, warmup):
    """The Qwen3-235B mixed batch: one prefill call of 16 one-row decode queries at 32768 keys (the
    first 16 sequences of w) and 4 fresh 512-token prompts, under the automatic prefill grid (the
    decode rows run one workgroup per split) and under in-workgroup folds."""
    shape = w.shape
    nq = 512
    lens_p = [nq] * 4
    layout_p = wl.layout_pages(21, lens_p, shape.P)
    kp = torch.zeros((layout_p.num_pages, shape.Hkv, shape.d // 8, shape.P, 8), dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros((layout_p.num_pages, shape.Hkv, shape.d, shape.P), dtype=torch.bfloat16, device=DEV)
    # One pool holds both: the prompts' pages are placed after the decode world's pages.
    base = w.layout.num_pages
    kk = torch.cat([w.k, kp])
    vv = torch.cat([w.v, vp])
    g = torch.Generator(device=DEV)
    g.manual_seed(SEED + 23)
    for b in range(4):
        sl = torch.as_tensor(layout_p.slots(b, 0, nq, shape.P) + base * shape.P, device=DEV)
        ia.ia_kv_append(w.ctx, torch.randn((nq, shape.Hkv, shape.d), generator=g, device=DEV).to(torch.bfloat16),
                        torch.randn((nq, shape.Hkv, shape.d), generator=g, device=DEV).to(torch.bfloat16), sl, kk, vv)
    width = max(w.layout.block_table.shape[1], layout_p.block_table.shape[1])
    bt = np.full((20, width), -1, np.int32)
    bt[:16, :w.layout.block_table.shape[1]] = w.layout.block_table[:16]
    btp = layout_p.block_table.copy()
    btp[btp >= 0] += base
    bt[16:, :btp.shape[1]] = btp
    q = torch.cat([w.q[:16], torch.randn((4 * nq, shape.Hq, shape.d), generator=g, device=DEV).to(torch.bfloat16)])
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum([1] * 16 + [nq] * 4)]).astype(np.int32), device=DEV)
    sl = torch.as_tensor(np.array([32768] * 16 + [nq] * 4, np.int32), device=DEV)
    btd = torch.as_tensor(bt, device=DEV)
    o = torch.empty_like(q)
    ws = prefill_workspace(w.ctx, 20, q.shape[0], nq, 32768)
    stream = torch.cuda.current_stream()

    flops = 4.0 * shape.d * shape.Hq * (16 * 32768 + 4 * nq * (nq + 1) / 2)
    out = {}
    for name, grid in (("auto", ia.IA_PREFILL_AUTO), ("fold", ia.IA_PREFILL_FOLD)):
        ctx = w.ctx if grid == ia.IA_PREFILL_AUTO else make_ctx(shape, prefill_grid=grid)

        def mixed():
            ia.ia_paged_attn_prefill(ctx, q, cu, sl, kk, vv, btd, nq, 32768, o, workspace=ws, stream=stream)

        ms = _timed(mixed, steps, warmup)
        out[name] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                     "decode_kv_gbs": round(w.kv_bytes(range(16)) / ms / 1e6, 1)}
    del kk, vv, kp, vp
    torch.cuda.empty_cache()
    return out


def qwen235_points(steps, warmup):
    """Qwen3-235B-A22B attention shape (64 query / 4 KV heads, head_dim 128, bf16): decode at 32768
    context for batch 1 / 16 / 64 -- the automatic kernel choice, and the cost of invariance with the
    split kernel pinned (fixed 2048-token splits against the split-by-count variant, same kernel) --
    and the mixed batch: 16 decode rows at 32768 context co-batched with 4 fresh 512-token prefill
    chunks in one prefill call."""
    shape = wl.QWEN3_235B
    w = DecodeWorld(shape, [32768] * 64, gpu_values=True)
    ctxs = {"auto": w.ctx, "split_fixed": make_ctx(shape, decode_kernel=ia.IA_DECODE_SPLIT),
            "split_by_count": make_ctx(shape, by_count=True, decode_kernel=ia.IA_DECODE_SPLIT)}
    out = {}
    for B in (1, 16, 64):
        kb = w.kv_bytes(range(B))
        row = {}
        for name, ctx in ctxs.items():
            _, d_ms = time_steps(DecodeRunner(w, range(B), ctx), steps, warmup, with_append=False)
            _, dc_ms = time_steps(DecodeRunner(w, range(B), ctx), max(5, steps // 5), 3, with_append=False, flush=True)
            row[name] = {"decode_ms": round(d_ms, 4), "gbs": round(kb / d_ms / 1e6, 1),
                         "hbm_frac": round(kb / d_ms / 1e6 / HBM_PEAK_GBS, 4), "decode_ms_cold": round(dc_ms, 4),
                         "gbs_cold": round(kb / dc_ms / 1e6, 1)}
        row["fixed_over_by_count_time_same_kernel"] = round(row["split_fixed"]["decode_ms"] /
                                                            row["split_by_count"]["decode_ms"], 3)
        out[f"B{B}"] = row
        log(f"qwen3-235b 32k B={B}: {row}")
    # Mixed batch: one prefill call of 16 one-row decode queries (n = 32768) + 4 fresh 512-token prompts.
    mixed = qwen235_mixed_call(w, steps, warmup)
    out["mixed_16x32k_decode_4x512_prefill"] = mixed["auto"]
    out["mixed_16x32k_decode_4x512_prefill_folds"] = mixed["fold"]
    log(f"qwen3-235b mixed: {mixed}")
    del w
    torch.cuda.empty_cache()
    return out


def llama70_points(steps, warmup):
    """Llama-3.1-70B-shaped attention (64 query / 8 KV heads, head_dim 128): 128 sequences on a shared
    16384-token prefix (1024 refcounted pages) plus private suffixes of 256-4096 tokens, block tables
    of 8192 entries (131072 keys), bf16 pages and fp8 e4m3 pages with static per-head scales; and one
    sequence at 131072 keys.  Logical KV bytes (what every sequence reads) against the distinct pages'
    bytes; DRAM bytes of the same launch come from the profile's FETCH_SIZE counters."""
    shape = wl.LLAMA31_70B
    lens = _shared_prefix_lens()
    out = {}
    for fp8 in (False, True):
        w = DecodeWorld(shape, lens, fp8=fp8, shared_prefix=16384, width=8192, gpu_values=True)
        # The sequences share their prefix pages: the deployment's hint is IA_KV_HINT_CACHED, so one
        # cached copy of a shared page serves every sequence; the automatic hint (which streams a
        # launch this large) is timed beside it.
        cached = make_ctx(shape, fp8=fp8, kv_cache_hint=ia.IA_KV_HINT_CACHED)
        _, d_ms = time_steps(DecodeRunner(w, range(128), cached), steps, warmup, with_append=False)
        _, dc_ms = time_steps(DecodeRunner(w, range(128), cached), max(5, steps // 5), 3, with_append=False,
                              flush=True)
        _, da_ms = time_steps(DecodeRunner(w, range(128)), steps, warmup, with_append=False)
        bpt = shape.Hkv * shape.d * 2 * (1 if fp8 else 2)
        key = "fp8" if fp8 else "bf16"
        out[key] = {"kv_cache_hint": "cached", "decode_ms": round(d_ms, 4),
                    "logical_gbs": round(w.kv_bytes() / d_ms / 1e6, 1),
                    "distinct_page_gbs": round(w.distinct_pages * shape.P * bpt / d_ms / 1e6, 1),
                    "decode_ms_cold": round(dc_ms, 4), "logical_gbs_cold": round(w.kv_bytes() / dc_ms / 1e6, 1),
                    "logical_bytes": w.kv_bytes(), "distinct_page_bytes": w.distinct_pages * shape.P * bpt,
                    "auto_hint_decode_ms": round(da_ms, 4),
                    "auto_hint_logical_gbs": round(w.kv_bytes() / da_ms / 1e6, 1)}
        log(f"llama70b shared prefix {key}: {out[key]}")
        del w
        torch.cuda.empty_cache()
    w = DecodeWorld(shape, [131072], width=8192, gpu_values=True)
    _, d_ms = time_steps(DecodeRunner(w, range(1)), steps, warmup, with_append=False)
    out["B1_131072"] = {"decode_ms": round(d_ms, 4), "gbs": round(w.kv_bytes() / d_ms / 1e6, 1)}
    log(f"llama70b B=1 at 131072: {out['B1_131072']}")
    del w
    torch.cuda.empty_cache()
    return out


def _timed(fn, steps, warmup):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def prefill_chunked(steps, warmup):
    """Qwen3-8B-shaped prefill of 8 prompts x 4096 tokens in chunks of 64 / 256 / 1024 tokens (chunk k of
    every prompt in one call, key length = the chunk's end), and its second half alone over a cached
    2048-token prefix; TFLOP/s over all the calls of a pass (4 d Hq sum over rows of p + 1)."""
    shape = wl.QWEN3_8B
    n, B = 4096, 8
    seqs, layout, ctx, k, v = _prefill_world(shape, [n] * B, 5)
    q = torch.cat([s.q(SEED, shape, 0, n) for s in seqs]).to(DEV).view(B, n, shape.Hq, shape.d)
    bt = torch.as_tensor(layout.block_table, device=DEV)
    stream = torch.cuda.current_stream()

    def calls(p_pairs):
        prepared = []
        for p0, p1 in p_pairs:
            qc = q[:, p0:p1].reshape(-1, shape.Hq, shape.d).contiguous()
            cu = torch.as_tensor(np.arange(0, B * (p1 - p0) + 1, p1 - p0, dtype=np.int32), device=DEV)
            sl = torch.as_tensor(np.full(B, p1, np.int32), device=DEV)
            prepared.append((qc, cu, sl, torch.empty_like(qc), p1 - p0, p1,
                             prefill_workspace(ctx, B, qc.shape[0], p1 - p0, p1)))
        return prepared

    def run(prepared):
        for qc, cu, sl, o, ql, kl, ws in prepared:
            ia.ia_paged_attn_prefill(ctx, qc, cu, sl, k, v, bt, ql, kl, o, workspace=ws, stream=stream)

    def flops(p0, p1):
        return 4.0 * shape.d * shape.Hq * B * sum(p + 1 for p in range(p0, p1))

    out = {}
    for budget in (64, 256, 1024, n):
        pairs = [(c0, min(n, c0 + budget)) for c0 in range(0, n, budget)]
        prep = calls(pairs)
        ms = _timed(lambda: run(prep), max(3, steps // 10), 2)
        fl = sum(flops(a, b) for a, b in pairs)
        key = "whole" if budget == n else f"chunks_{budget}"
        out[key] = {"calls_per_pass": len(pairs), "ms_per_pass": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                    "frac_of_bf16_peak": round(fl / ms / 1e9 / BF16_PEAK_TFLOPS, 4)}
        log(f"prefill {key}: {out[key]}")
    prep = calls([(n // 2, n)])
    ms = _timed(lambda: run(prep), max(5, steps // 5), 3)
    fl = flops(n // 2, n)
    out["cached_prefix_2048_suffix_2048"] = {"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                                             "frac_of_bf16_peak": round(fl / ms / 1e9 / BF16_PEAK_TFLOPS, 4)}
    log(f"prefill cached prefix: {out['cached_prefix_2048_suffix_2048']}")
    del k, v, q
    torch.cuda.empty_cache()
    return out


def manifest(config: dict):
    """Where the numbers came from: git commit (or the one recorded at build time when the tree has no
    .git), a hash of the library's sources as they ran, the GPU's architecture, and a config hash."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "invariant_attention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    build_sha = None
    try:
        with open(os.path.join(ROOT, "invariant_attention_amd", "build_info.json")) as f:
            build_sha = json.load(f).get("git")
    except (OSError, ValueError):
        pass
    props = torch.cuda.get_device_properties(0)
    return {"git": git_sha() or build_sha, "git_at_build": build_sha, "sources_sha256": h.hexdigest()[:16],
            "config_sha256": hashlib.sha256(json.dumps(config, sort_keys=True).encode()).hexdigest()[:16],
            "torch": torch.__version__, "hip": torch.version.hip, "device": torch.cuda.get_device_name(0),
            "gfx_arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count,
            "seed": SEED, "host_threads": os.cpu_count(), "cpu": cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=256)
    ap.add_argument("--decode-only", action="store_true", help="time the headline batch only (for profilers)")
    ap.add_argument("--copy-probe", action="store_true", help="run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true", help="time the prefill workload only (for profilers)")
    ap.add_argument("--layer-only", action="store_true", help="time the layer operators only (for profilers)")
    ap.add_argument("--mixed-only", action="store_true",
                    help="time the Qwen3-235B mixed prefill call only, automatic grid and folds (for profilers)")
    ap.add_argument("--shared-prefix-only", action="store_true",
                    help="time the Llama-3.1-70B shared-prefix decode only (for profilers)")
    ap.add_argument("--summarize-shared-prefix-profile", nargs=2, metavar=("TRACE_DIR", "PMC_DIR"))
    ap.add_argument("--summarize-profile", nargs=2, metavar=("TRACE_DIR", "PMC_DIR"))
    ap.add_argument("--summarize-prefill-profile", nargs=2, metavar=("TRACE_DIR", "PMC_DIR"))
    ap.add_argument("--summarize-spread-profile", metavar="TRACE_DIR")
    ap.add_argument("--summarize-mixed-profile", metavar="TRACE_DIR")
    ap.add_argument("--summarize-layer-profile", nargs=2, metavar=("TRACE_DIR", "LAYER_JSON"))
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(*args.summarize_profile)
        return
    if args.summarize_prefill_profile:
        summarize_prefill_profile(*args.summarize_prefill_profile)
        return
    if args.summarize_shared_prefix_profile:
        summarize_shared_prefix_profile(*args.summarize_shared_prefix_profile)
        return
    if args.summarize_spread_profile:
        summarize_spread_profile(args.summarize_spread_profile)
        return
    if args.summarize_mixed_profile:
        summarize_mixed_profile(args.summarize_mixed_profile)
        return
    if args.summarize_layer_profile:
        summarize_layer_profile(*args.summarize_layer_profile)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only; there is no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ia.load()
    if args.copy_probe:
        print(json.dumps({"copy_probe": copy_gbs(reps=args.steps)}), flush=True)
        return
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_tflops(args.steps, args.warmup)}), flush=True)
        return
    if args.layer_only:
        print(json.dumps({"layer_ops": layer_ops(args.steps, args.warmup)}), flush=True)
        return
    if args.mixed_only:
        w = DecodeWorld(wl.QWEN3_235B, [32768] * 16, gpu_values=True)
        print(json.dumps({"qwen235_mixed": qwen235_mixed_call(w, args.steps, args.warmup)}), flush=True)
        return
    if args.shared_prefix_only:
        shape = wl.LLAMA31_70B
        w = DecodeWorld(shape, _shared_prefix_lens(), shared_prefix=16384, width=8192, gpu_values=True)
        ctx = make_ctx(shape, kv_cache_hint=ia.IA_KV_HINT_CACHED)
        _, d_ms = time_steps(DecodeRunner(w, range(128), ctx), args.steps, args.warmup, with_append=False)
        print(json.dumps({"shared_prefix_decode_ms": round(d_ms, 4),
                          "logical_gbs": round(w.kv_bytes() / d_ms / 1e6, 1)}), flush=True)
        return
    shape = wl.LLAMA3_8B
    lens = wl.uniform_lens(SEED, args.batch, 512, 8192)
    log(f"decode workload: llama3-8b shape, B={args.batch}, {sum(lens)} tokens")
    world = DecodeWorld(shape, lens, keep_host=not (args.no_cpu_baseline or args.decode_only))
    head = DecodeRunner(world, range(args.batch))
    torch.cuda.synchronize()
    step_ms, dec_ms = time_steps(head, args.steps, args.warmup)
    kvb = world.kv_bytes()
    value = kvb / (step_ms * 1e-3) / 1e9
    dec_gbs = kvb / (dec_ms * 1e-3) / 1e9
    pct = {f"p{q}": round(float(np.percentile(time_steps.last_calls, q)), 4) for q in (10, 50, 90)}
    log(f"B={args.batch}: step {step_ms:.4f} ms ({value:.0f} GB/s), decode call {dec_ms:.4f} ms ({dec_gbs:.0f} GB/s), "
        f"call ms percentiles {pct}")
    result = {
        "metric": "batch-invariant paged-attn decode KV GB/s (% HBM peak) + bitwise invariance rate",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) K/V/Q, random page placement)",
        "config": {"workload": "llama3-8b-shaped paged decode step (kv_append + decode), batch 256, "
                               "contexts uniform in [512, 8192]",
                   "batch": args.batch, "q_heads": shape.Hq, "kv_heads": shape.Hkv, "head_dim": shape.d,
                   "page_size": shape.P, "split_tokens": shape.S, "tokens": int(sum(lens)), "kv_dtype": "bf16"},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"kernel": "decode_split_kernel (with its split merge: one ia_paged_attn_decode call)",
                     "bound": "hbm", "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
                     "algorithmic_bytes_per_launch": kvb, "avg_launch_ms": round(dec_ms, 4),
                     "launch_ms_percentiles": pct},
    }
    if not args.decode_only:
        result["copy_reference"] = copy_gbs()
        result["stream_read_reference"] = stream_read_reference()
        result["read_reference"] = read_gbs()
        log(f"plain copy: {result['copy_reference']}, stream read: {result['stream_read_reference']}, "
            f"torch sum: {result['read_reference']}")
        result["kv_append_prefill_size"] = kv_append_prefill_size()
        log(f"kv_append at prefill size: {result['kv_append_prefill_size']}")
        batches, by_count, same_kernel = {}, {}, {}
        bc_ctx = make_ctx(shape, by_count=True)
        split_fixed = make_ctx(shape, decode_kernel=ia.IA_DECODE_SPLIT)
        split_bc = make_ctx(shape, by_count=True, decode_kernel=ia.IA_DECODE_SPLIT)
        for B in (1, 8, 64, args.batch):
            s_ms, d_ms = time_steps(DecodeRunner(world, range(B)), args.steps, args.warmup)
            _, dc_ms = time_steps(DecodeRunner(world, range(B)), args.steps, args.warmup, flush=True)
            kb = world.kv_bytes(range(B))
            batches[str(B)] = {"step_ms": round(s_ms, 4), "decode_ms": round(d_ms, 4),
                               "gbs": round(kb / (s_ms * 1e-3) / 1e9, 1), "decode_ms_cold": round(dc_ms, 4),
                               "decode_gbs_cold": round(kb / (dc_ms * 1e-3) / 1e9, 1)}
            s2, d2 = time_steps(DecodeRunner(world, range(B), bc_ctx), args.steps, args.warmup)
            _, d2c = time_steps(DecodeRunner(world, range(B), bc_ctx), args.steps, args.warmup, flush=True)
            by_count[str(B)] = {"step_ms": round(s2, 4), "gbs": round(kb / (s2 * 1e-3) / 1e9, 1),
                                "fixed_over_by_count_time": round(s_ms / s2, 3), "decode_ms_cold": round(d2c, 4),
                                "fixed_over_by_count_time_cold": round(dc_ms / d2c, 3)}
            # The cost of invariance on one kernel: both split policies on the split kernel.
            _, f_ms = time_steps(DecodeRunner(world, range(B), split_fixed), args.steps, args.warmup)
            _, c_ms = time_steps(DecodeRunner(world, range(B), split_bc), args.steps, args.warmup)
            same_kernel[str(B)] = {"fixed_decode_ms": round(f_ms, 4), "by_count_decode_ms": round(c_ms, 4),
                                   "fixed_gbs": round(kb / (f_ms * 1e-3) / 1e9, 1),
                                   "by_count_gbs": round(kb / (c_ms * 1e-3) / 1e9, 1),
                                   "fixed_over_by_count_time": round(f_ms / c_ms, 3)}
            log(f"B={B}: fixed {batches[str(B)]['gbs']} GB/s, split-by-count {by_count[str(B)]['gbs']} GB/s; "
                f"split kernel for both: {same_kernel[str(B)]}")
        result["batches"] = batches
        result["split_by_count"] = by_count
        result["cost_of_invariance_split_kernel"] = same_kernel
        # The same decode call with the caches flushed before each call (no K/V or table data left
        # from the previous step), beside the steady-state figure above.
        cold_ms = batches[str(args.batch)]["decode_ms_cold"]
        result["roofline"]["cache_flushed"] = {"avg_launch_ms": cold_ms,
                                               "achieved": round(kvb / (cold_ms * 1e-3) / 1e9, 2),
                                               "frac": round(kvb / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        # The bitwise-equivalent decode kernels at small batches: the split kernel alone, the spread
        # kernels alone (the automatic choice runs them up to 64 split units) and the wide kernel.
        kern = {}
        for name, kid in (("split", ia.IA_DECODE_SPLIT), ("spread", ia.IA_DECODE_SPREAD), ("wide", ia.IA_DECODE_WIDE)):
            kctx = make_ctx(shape, decode_kernel=kid)
            kern[name] = {}
            for B in (1, 8, 16, 32, 64):
                if name == "wide" and B not in (1, 8, 64):
                    continue
                s_ms, d_ms = time_steps(DecodeRunner(world, range(B), kctx), args.steps, args.warmup)
                kern[name][str(B)] = {"decode_ms": round(d_ms, 4),
                                      "decode_gbs": round(world.kv_bytes(range(B)) / (d_ms * 1e-3) / 1e9, 1)}
                if B in (1, 8):
                    _, dc = time_steps(DecodeRunner(world, range(B), kctx), args.steps, args.warmup, flush=True)
                    kern[name][str(B)]["decode_ms_cold"] = round(dc, 4)
            log(f"{name} decode kernel: {kern[name]}")
        result["decode_kernels"] = kern
        probes = [0, 1, 37, 100, 200, args.batch - 1]
        eq, tot = invariance_pairs(world, world.ctx, probes)
        eq_c, tot_c = invariance_pairs(world, bc_ctx, probes)
        var = invariance_variations(lens)
        var["batch_composition"] = (eq, tot)
        eq_all, tot_all = sum(e for e, _ in var.values()), sum(t for _, t in var.values())
        result["invariance_rate"] = round(eq_all / tot_all, 6)
        result["invariance_pairs"] = f"{eq_all}/{tot_all}"
        result["invariance_by_variation"] = {k: f"{e}/{t}" for k, (e, t) in var.items()}
        result["split_by_count_invariance_rate"] = round(eq_c / tot_c, 6)
        log(f"invariance: fixed {eq_all}/{tot_all} {result['invariance_by_variation']}, split-by-count {eq_c}/{tot_c}")
    if not args.no_cpu_baseline and not args.decode_only:
        result["cpu_baseline"] = cpu_baseline(world)
        log(f"cpu baseline: {result['cpu_baseline']}")
    del world, head
    torch.cuda.empty_cache()
    if not args.decode_only:
        result["prefill"] = prefill_tflops(max(10, args.steps // 4), 10)
        log(f"prefill: {result['prefill']}")
        result["prefill_chunked"] = prefill_chunked(args.steps, args.warmup)
        result["qwen3_235b"] = qwen235_points(args.steps, args.warmup)
        result["llama31_70b_shared_prefix"] = llama70_points(args.steps, args.warmup)
        result["layer_ops"] = layer_ops(max(3, args.steps // 4), 2)
    result["manifest"] = manifest(result["config"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
