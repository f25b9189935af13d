"""GPU-side helpers for the tests and the bench: put synthetic sequences into device page pools
through the library's kv_append and run its attention entry points (all through the C ABI)."""
from __future__ import annotations

import numpy as np
import torch

from invariant_attention_amd import binding as ia
from synth import workloads as wl

DEV = "cuda"
TOL_ABS, TOL_REL = 2e-3, 1e-2


def within_tolerance(gpu: torch.Tensor, ref: np.ndarray):
    """Element-wise |gpu - ref| <= 2e-3 + 1e-2 |ref|; returns (ok, max_abs_err, worst_ratio)."""
    g = gpu.detach().to("cpu", torch.float64).numpy()
    err = np.abs(g - ref)
    bound = TOL_ABS + TOL_REL * np.abs(ref)
    return bool(np.all(err <= bound)), float(err.max(initial=0.0)), float((err / bound).max(initial=0.0))


def make_ctx(shape: wl.AttnShape, fp8=False, by_count=False, split_tokens=None, window=0,
             decode_kernel=ia.IA_DECODE_AUTO, kv_cache_hint=ia.IA_KV_HINT_AUTO, prefill_grid=ia.IA_PREFILL_AUTO):
    cfg = ia.make_config(shape.Hq, shape.Hkv, shape.d, page_size=shape.P,
                         split_tokens=shape.S if split_tokens is None else split_tokens,
                         kv_dtype=ia.IA_KV_FP8_E4M3 if fp8 else ia.IA_KV_BF16,
                         split_policy=ia.IA_SPLIT_BY_COUNT if by_count else ia.IA_SPLIT_FIXED,
                         sm_scale=shape.scale, sliding_window=window, decode_kernel=decode_kernel,
                         kv_cache_hint=kv_cache_hint, prefill_grid=prefill_grid)
    return ia.Context(cfg)


class DevicePages:
    """Device K/V page pools for one shape (bf16 or fp8 codes) plus static fp8 scales."""

    def __init__(self, shape: wl.AttnShape, num_pages: int, fp8=False, k_scale=None, v_scale=None):
        self.shape = shape
        self.fp8 = fp8
        dt = torch.uint8 if fp8 else torch.bfloat16
        self.k = torch.zeros((num_pages, shape.Hkv, shape.d // 8, shape.P, 8), dtype=dt, device=DEV)
        self.v = torch.zeros((num_pages, shape.Hkv, shape.d, shape.P), dtype=dt, device=DEV)
        self.k_scale = torch.as_tensor(k_scale, dtype=torch.float32, device=DEV) if fp8 else None
        self.v_scale = torch.as_tensor(v_scale, dtype=torch.float32, device=DEV) if fp8 else None

    def append(self, ctx, k_rows: torch.Tensor, v_rows: torch.Tensor, slots: np.ndarray, stream=None):
        k = k_rows.to(DEV).contiguous()
        v = v_rows.to(DEV).contiguous()
        sl = torch.as_tensor(np.ascontiguousarray(slots, dtype=np.int64), device=DEV)
        ia.ia_kv_append(ctx, k, v, sl, self.k, self.v, self.k_scale, self.v_scale, stream=stream)

    def host_bits(self):
        """Page pools as host uint16 (bf16 bits) / uint8 arrays, for bit comparison."""
        if self.fp8:
            return self.k.cpu().numpy(), self.v.cpu().numpy()
        return (self.k.cpu().view(torch.int16).numpy().view(np.uint16),
                self.v.cpu().view(torch.int16).numpy().view(np.uint16))


def fill_sequences(ctx, pages: DevicePages, seqs, layout: wl.PageLayout, seed: int, upto=None, chunk=65536):
    """kv_append every position (< upto[b]) of every sequence, at most `chunk` rows per call."""
    shape = pages.shape
    for b, s in enumerate(seqs):
        hi = s.n if upto is None else upto[b]
        for p0 in range(0, hi, chunk):
            p1 = min(hi, p0 + chunk)
            pages.append(ctx, s.k(seed, shape, p0, p1), s.v(seed, shape, p0, p1), layout.slots(b, p0, p1, shape.P))


def decode(ctx, pages: DevicePages, q: torch.Tensor, layout: wl.PageLayout, seq_lens, max_seq_len=None,
           stream=None, block_table=None, ws=None):
    shape = pages.shape
    B = len(seq_lens)
    qd = q.to(DEV).contiguous()
    sl = torch.as_tensor(np.asarray(seq_lens, dtype=np.int32), device=DEV)
    bt = torch.as_tensor(layout.block_table, device=DEV) if block_table is None else block_table
    msl = int(max(seq_lens)) if max_seq_len is None else int(max_seq_len)
    out = torch.empty((B, shape.Hq, shape.d), dtype=torch.bfloat16, device=DEV)
    if ws is None:
        ws = torch.empty(max(1, ia.ia_decode_workspace_bytes(ctx, B, msl)), dtype=torch.uint8, device=DEV)
    ia.ia_paged_attn_decode(ctx, qd, pages.k, pages.v, bt, sl, msl, out, ws, pages.k_scale, pages.v_scale,
                            stream=stream)
    return out


def prefill(ctx, pages: DevicePages, q: torch.Tensor, cu: np.ndarray, layout: wl.PageLayout, seq_lens,
            max_seq_len=None, max_q_len=None, stream=None, workspace_bytes=None):
    """workspace_bytes: the workspace passed (default: the size the library asks for)."""
    shape = pages.shape
    qd = q.to(DEV).contiguous()
    cu_d = torch.as_tensor(np.asarray(cu, dtype=np.int32), device=DEV)
    sl = torch.as_tensor(np.asarray(seq_lens, dtype=np.int32), device=DEV)
    bt = torch.as_tensor(layout.block_table, device=DEV)
    q_lens = np.diff(np.asarray(cu))
    mql = int(q_lens.max(initial=0)) if max_q_len is None else int(max_q_len)
    msl = int(max(seq_lens)) if max_seq_len is None else int(max_seq_len)
    out = torch.empty((q.shape[0], shape.Hq, shape.d), dtype=torch.bfloat16, device=DEV)
    nws = (ia.ia_prefill_workspace_bytes(ctx, len(q_lens), int(q.shape[0]), mql, msl) if workspace_bytes is None
           else workspace_bytes)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV) if nws else None
    ia.ia_paged_attn_prefill(ctx, qd, cu_d, sl, pages.k, pages.v, bt, mql, msl, out, pages.k_scale,
                             pages.v_scale, workspace=ws, stream=stream)
    return out


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy()


class MiniEngine:
    """An attention-only stand-in for an inference engine.  The library's page pool (C ABI) decides
    which cached pages a new sequence reuses and where each computed position's K/V goes;
    kv_append writes them; prefill and decode read them through the pool's block table.  No model:
    a position's K/V/Q rows come from the seeded generators."""

    def __init__(self, shape: wl.AttnShape, num_pages: int, seed: int = 0, fp8=False, scales=(None, None),
                 flags: int = 0, ctx=None):
        self.shape = shape
        self.seed = seed
        self.num_pages = num_pages
        self.pool = ia.Pool(num_pages, shape.P, flags)
        self.pages = DevicePages(shape, num_pages, fp8, *scales)
        self.ctx = make_ctx(shape, fp8=fp8) if ctx is None else ctx
        self.hist = {}  # handle -> positions that have a token in the pool's history

    def begin(self, seq: wl.Sequence, n_prompt: int | None = None):
        """Starts seq with its first n_prompt tokens; returns (handle, cached positions)."""
        n_prompt = seq.n if n_prompt is None else n_prompt
        h, cached = ia.ia_seq_begin(self.pool, seq.tokens(0, n_prompt))
        self.hist[h.value] = n_prompt
        return h, cached

    def _layout(self, h) -> wl.PageLayout:
        bt = np.array(ia.ia_seq_block_table(h), dtype=np.int32)
        return wl.PageLayout(self.num_pages, bt[None, :], [bt.astype(np.int64)])

    def _append(self, seq, h, p0, p1):
        slots = np.array(ia.ia_seq_reserve(self.pool, h, p1 - p0), dtype=np.int64)
        self.pages.append(self.ctx, seq.k(self.seed, self.shape, p0, p1), seq.v(self.seed, self.shape, p0, p1),
                          slots)

    def prefill(self, seq, h, p0: int, p1: int) -> torch.Tensor:
        """Computes positions [p0, p1) (the next ones of the history) in one prefill call."""
        assert ia.ia_seq_len(h) == p0 and p1 <= self.hist[h.value]
        self._append(seq, h, p0, p1)
        out = prefill(self.ctx, self.pages, seq.q(self.seed, self.shape, p0, p1), np.array([0, p1 - p0]),
                      self._layout(h), [p1])
        ia.ia_seq_commit(self.pool, h, p1 - p0)
        return out

    def decode(self, seq, h, p: int) -> torch.Tensor:
        """Computes position p (the next one) with the decode entry point, appending its token to
        the history first if it is not part of the prompt."""
        assert ia.ia_seq_len(h) == p
        if p >= self.hist[h.value]:
            ia.ia_seq_append_tokens(self.pool, h, seq.tokens(p, p + 1))
            self.hist[h.value] = p + 1
        self._append(seq, h, p, p + 1)
        out = decode(self.ctx, self.pages, seq.q(self.seed, self.shape, p, p + 1), self._layout(h), [p + 1])
        ia.ia_seq_commit(self.pool, h, 1)
        return out

    def end(self, h) -> None:
        ia.ia_seq_end(self.pool, h)
        self.hist.pop(h.value, None)
