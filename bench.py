#!/usr/bin/env python3
"""Benchmark: batch-invariant paged-attention decode on one MI355X.

A step is one decode step of the Llama-3-8B-shaped workload (32 query / 8 KV heads, head_dim
128, bf16 pages of 16 tokens, fixed 2048-token splits, contexts uniform in [512, 8192]): the
step's new K/V rows are written into their page slots (kv_append) and every sequence's query
row attends its whole paged context (decode split kernel + ascending split merge).  The timed
region starts with every input resident in HBM.

`value` is decode KV-read throughput at batch 256: the algorithmic KV bytes of the step
(sum_b n_b * Hkv * d * 2 tensors * 2 bytes -- each sequence's K and V read once per KV head)
divided by the step time.  The JSON line also carries the roofline of the decode kernels
(their own duration, from HIP events on the launch stream), the batch sizes 1/8/64, the
split-by-count comparison variant (the cost of invariance), a bitwise invariance rate measured
in the same run, prefill TFLOP/s, and the fp64 CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""
from __future__ import annotations

import argparse
import json
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


class DecodeWorld:
    """The decode workload resident on the GPU: pages, tables, queries, new-token rows, slots."""

    def __init__(self, shape: wl.AttnShape, lens, fp8=False):
        self.shape = shape
        self.lens = [int(n) for n in lens]
        self.B = len(self.lens)
        self.seqs = wl.make_sequences(self.lens)
        self.layout = wl.layout_pages(3, self.lens, shape.P)
        self.ctx = make_ctx(shape)
        dt = torch.uint8 if fp8 else torch.bfloat16
        npg = self.layout.num_pages
        self.k = torch.zeros((npg, shape.Hkv, shape.d // 8, shape.P, 8), dtype=dt, device=DEV)
        self.v = torch.zeros((npg, shape.Hkv, shape.d, shape.P), dtype=dt, device=DEV)
        t0 = time.time()
        qs, knew, vnew, slots = [], [], [], []
        for b, s in enumerate(self.seqs):
            kr = s.k(SEED, shape)
            vr = s.v(SEED, shape)
            sl = torch.as_tensor(self.layout.slots(b, 0, s.n, shape.P), device=DEV)
            ia.ia_kv_append(self.ctx, kr.to(DEV), vr.to(DEV), sl, self.k, self.v)
            qs.append(s.q(SEED, shape, s.n - 1, s.n))
            knew.append(kr[-1:])
            vnew.append(vr[-1:])
            slots.append(self.layout.slots(b, s.n - 1, s.n, shape.P))
        torch.cuda.synchronize()
        log(f"  filled {self.B} sequences ({sum(self.lens)} tokens) in {time.time() - t0:.1f}s")
        self.q = torch.cat(qs).to(DEV)
        self.k_new = torch.cat(knew).to(DEV)
        self.v_new = torch.cat(vnew).to(DEV)
        self.slots = torch.as_tensor(np.concatenate(slots), device=DEV)
        self.bt = torch.as_tensor(self.layout.block_table, device=DEV)
        self.seq_lens = torch.as_tensor(np.array(self.lens, np.int32), device=DEV)
        self.max_len = max(self.lens)

    def kv_bytes(self, idx=None) -> int:
        lens = self.lens if idx is None else [self.lens[i] for i in idx]
        return int(sum(lens)) * self.shape.Hkv * self.shape.d * 2 * 2


def make_ctx(shape, by_count=False):
    return ia.Context(ia.make_config(shape.Hq, shape.Hkv, shape.d, page_size=shape.P, split_tokens=shape.S,
                                     split_policy=ia.IA_SPLIT_BY_COUNT if by_count else ia.IA_SPLIT_FIXED,
                                     sm_scale=shape.scale))


class DecodeRunner:
    """One batch (a prefix of the world's sequences) ready to step."""

    def __init__(self, world: DecodeWorld, B: int, ctx=None):
        self.w = world
        self.B = B
        self.ctx = world.ctx if ctx is None else ctx
        self.q = world.q[:B].contiguous()
        self.bt = world.bt[:B].contiguous()
        self.sl = world.seq_lens[:B].contiguous()
        self.k_new = world.k_new[:B].contiguous()
        self.v_new = world.v_new[:B].contiguous()
        self.slots = world.slots[:B].contiguous()
        self.max_len = max(world.lens[:B])
        self.out = torch.empty((B, world.shape.Hq, world.shape.d), dtype=torch.bfloat16, device=DEV)
        nb = ia.ia_decode_workspace_bytes(self.ctx, B, self.max_len)
        self.ws = torch.empty(nb, dtype=torch.uint8, device=DEV)

    def append(self, stream):
        ia.ia_kv_append(self.ctx, self.k_new, self.v_new, self.slots, self.w.k, self.w.v, stream=stream)

    def decode(self, stream):
        ia.ia_paged_attn_decode(self.ctx, self.q, self.w.k, self.w.v, self.bt, self.sl, self.max_len, self.out,
                                self.ws, stream=stream)


def time_steps(runner: DecodeRunner, steps: int, warmup: int):
    """Times `steps` steps (kv_append + decode).  Returns (step ms, decode-kernels ms) medians."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        runner.append(stream)
        runner.decode(stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(stream)
        runner.append(stream)
        e1.record(stream)
        runner.decode(stream)
        e2.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    step_ms = [e0.elapsed_time(e2) for e0, _, e2 in ev]
    dec_ms = [e1.elapsed_time(e2) for _, e1, e2 in ev]
    return float(np.median(step_ms)), float(np.median(dec_ms)), wall


def invariance_pairs(world: DecodeWorld, ctx, probes):
    """Bitwise comparisons of output rows across batch compositions: batch B vs alone, vs the
    first 8 and first 64, and vs the reversed batch.  Returns (equal, compared)."""
    B = world.B
    full = DecodeRunner(world, B, ctx)
    full.decode(None)
    ref = full.out.clone()
    eq = tot = 0

    def rows(idx):
        r = DecodeRunner.__new__(DecodeRunner)
        r.w, r.B, r.ctx = world, len(idx), ctx
        ii = torch.as_tensor(idx, device=DEV)
        r.q = world.q[ii].contiguous()
        r.bt = world.bt[ii].contiguous()
        r.sl = world.seq_lens[ii].contiguous()
        r.max_len = max(world.lens[i] for i in idx)
        r.out = torch.empty((len(idx), world.shape.Hq, world.shape.d), dtype=torch.bfloat16, device=DEV)
        r.ws = torch.empty(ia.ia_decode_workspace_bytes(ctx, len(idx), r.max_len), dtype=torch.uint8, device=DEV)
        r.decode(None)
        return r.out

    def cmp(out, idx):
        nonlocal eq, tot
        a = out.view(torch.int16).cpu().numpy().reshape(len(idx), -1)
        b = ref[torch.as_tensor(idx, device=DEV)].view(torch.int16).cpu().numpy().reshape(len(idx), -1)
        same = (a == b).all(axis=1)
        eq += int(same.sum())
        tot += len(idx)

    for p in probes:
        cmp(rows([p]), [p])
    for sub in (list(range(8)), list(range(64))):
        cmp(rows(sub), sub)
    rev = list(reversed(range(B)))
    cmp(rows(rev), rev)
    return eq, tot


def prefill_tflops(steps: int, warmup: int):
    """Whole prefill of 8 prompts x 4096 tokens (Qwen3-8B shape); flops = 4 d sum_rows (p+1) Hq."""
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
    stream = torch.cuda.current_stream()

    def run():
        ia.ia_paged_attn_prefill(ctx, q, cu, sl, k, v, bt, 4096, 4096, out, stream=stream)

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
    return {"workload": "qwen3-8b-prefill-8x4096", "ms": ms, "tflops": flops / ms / 1e9,
            "frac_of_bf16_peak": flops / ms / 1e9 / BF16_PEAK_TFLOPS}


def cpu_baseline(world: DecodeWorld, sample: int = 8):
    """The fp64 oracle (as it stands) on `sample` sequences of the batch, all heads, on the host."""
    from oracle import oracle
    shape = world.shape
    oracle.build(force=False)
    idx = list(range(sample))
    seqs = [world.seqs[i] for i in idx]
    lens = [s.n for s in seqs]
    layout = wl.layout_pages(9, lens, shape.P)
    kshape, vshape = oracle.kv_cache_shapes(layout.num_pages, shape.Hkv, shape.d, shape.P)
    kc, vc = np.zeros(kshape, np.uint16), np.zeros(vshape, np.uint16)
    for b, s in enumerate(seqs):
        oracle.kv_append(s.k(SEED, shape).view(torch.int16).numpy().view(np.uint16),
                         s.v(SEED, shape).view(torch.int16).numpy().view(np.uint16),
                         layout.slots(b, 0, s.n, shape.P), kc, vc, Hkv=shape.Hkv, d=shape.d, P=shape.P)
    q = torch.cat([s.q(SEED, shape, s.n - 1, s.n) for s in seqs]).view(torch.int16).numpy().view(np.uint16)
    cu = np.arange(sample + 1, dtype=np.int32)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.paged_attention(q, cu, np.array(lens, np.int32), kc, vc, layout.block_table, Hq=shape.Hq,
                           Hkv=shape.Hkv, d=shape.d, P=shape.P, scale=shape.scale, nthreads=threads)
    dt = time.perf_counter() - t0
    gbs = world.kv_bytes(idx) / dt / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{sample} of the batch-256 sequences ({sum(lens)} tokens, all 32 query heads), "
                      f"decode rows, fp64, {dt:.2f} s", "cpu": cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=256)
    ap.add_argument("--decode-only", action="store_true", help="time the headline batch only (for profilers)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (no multi-GPU path); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ia.load()
    shape = wl.LLAMA3_8B
    lens = wl.uniform_lens(SEED, args.batch, 512, 8192)
    log(f"decode workload: llama3-8b shape, B={args.batch}, {sum(lens)} tokens")
    world = DecodeWorld(shape, lens)
    head = DecodeRunner(world, args.batch)
    step_ms, dec_ms, wall_ms = time_steps(head, args.steps, args.warmup)
    kvb = world.kv_bytes()
    value = kvb / (step_ms * 1e-3) / 1e9
    dec_gbs = kvb / (dec_ms * 1e-3) / 1e9
    log(f"B={args.batch}: step {step_ms:.3f} ms ({value:.0f} GB/s), decode kernels {dec_ms:.3f} ms "
        f"({dec_gbs:.0f} GB/s), host wall {wall_ms:.3f} ms/step")
    result = {
        "metric": "batch-invariant paged-attn decode KV GB/s (% HBM peak) + bitwise invariance rate",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama3-8b-shaped decode (kv_append + decode)", "batch": args.batch,
                   "q_heads": shape.Hq, "kv_heads": shape.Hkv, "head_dim": shape.d, "page_size": shape.P,
                   "split_tokens": shape.S, "context": "uniform [512, 8192]", "tokens": int(sum(lens)),
                   "kv_dtype": "bf16"},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"kernel": "decode_split_kernel + decode_merge_kernel (one ia_paged_attn_decode call)",
                     "bound": "hbm", "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": kvb, "avg_launch_ms": round(dec_ms, 4)},
    }
    if not args.decode_only:
        batches = {}
        by_count = {}
        bc_ctx = make_ctx(shape, by_count=True)
        for B in (1, 8, 64, args.batch):
            r = DecodeRunner(world, B)
            s_ms, d_ms, _ = time_steps(r, args.steps, args.warmup)
            kb = world.kv_bytes(range(B))
            batches[str(B)] = {"step_ms": round(s_ms, 4), "decode_ms": round(d_ms, 4),
                               "gbs": round(kb / (s_ms * 1e-3) / 1e9, 1)}
            rc = DecodeRunner(world, B, bc_ctx)
            s2, d2, _ = time_steps(rc, args.steps, args.warmup)
            by_count[str(B)] = {"step_ms": round(s2, 4), "gbs": round(kb / (s2 * 1e-3) / 1e9, 1),
                                "fixed_over_by_count": round(s2 / s_ms, 3)}
            log(f"B={B}: fixed {batches[str(B)]['gbs']} GB/s, split-by-count {by_count[str(B)]['gbs']} GB/s")
        result["batches"] = batches
        result["split_by_count"] = by_count
        eq, tot = invariance_pairs(world, world.ctx, probes=[0, 1, 37, 100, 200, args.batch - 1])
        eq_c, tot_c = invariance_pairs(world, bc_ctx, probes=[0, 1, 37, 100, 200, args.batch - 1])
        result["invariance_rate"] = round(eq / tot, 6)
        result["invariance_pairs"] = f"{eq}/{tot}"
        result["split_by_count_invariance_rate"] = round(eq_c / tot_c, 6)
        log(f"invariance: fixed {eq}/{tot}, split-by-count {eq_c}/{tot_c}")
        result["prefill"] = prefill_tflops(max(3, args.steps // 4), 1)
        log(f"prefill: {result['prefill']}")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(world)
        log(f"cpu baseline: {result['cpu_baseline']}")
    result["manifest"] = {"git": git_sha(), "torch": torch.__version__, "hip": torch.version.hip,
                          "device": torch.cuda.get_device_name(0), "seed": SEED}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
