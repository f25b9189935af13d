"""Oracle-side helpers for the tests: lay synthetic sequences into host page pools with the
oracle's own scatter, and run the fp64 oracle.  Nothing here touches the HIP library."""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle
from synth import workloads as wl


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def host_pools(shape: wl.AttnShape, num_pages: int, fp8: bool = False):
    kshape, vshape = oracle.kv_cache_shapes(num_pages, shape.Hkv, shape.d, shape.P)
    dt = np.uint8 if fp8 else np.uint16
    return np.zeros(kshape, dtype=dt), np.zeros(vshape, dtype=dt)


def scatter_sequences(shape, seqs, layout, seed, kc, vc, fp8=False, k_scale=None, v_scale=None, upto=None):
    """Oracle kv_append of every position of every sequence (or positions < upto[b])."""
    for b, s in enumerate(seqs):
        hi = s.n if upto is None else upto[b]
        if hi <= 0:
            continue
        k = bits16(s.k(seed, shape, 0, hi))
        v = bits16(s.v(seed, shape, 0, hi))
        slots = layout.slots(b, 0, hi, shape.P)
        oracle.kv_append(k, v, slots, kc, vc, Hkv=shape.Hkv, d=shape.d, P=shape.P, kv_fp8=fp8,
                         k_scale=k_scale, v_scale=v_scale)


def queries(shape, seqs, seed, q_lens):
    """Packed bf16 queries for the last q_lens[b] positions of each sequence, and cu_q_lens."""
    parts = [s.q(seed, shape, s.n - ql, s.n) for s, ql in zip(seqs, q_lens)]
    q = torch.cat(parts, 0) if parts else torch.zeros((0, shape.Hq, shape.d), dtype=torch.bfloat16)
    cu = np.zeros(len(seqs) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    return q, cu


def run_oracle(shape, seqs, layout, seed, q_lens, fp8=False, k_scale=None, v_scale=None, split_tokens=0,
               nthreads=0, window=0):
    kc, vc = host_pools(shape, layout.num_pages, fp8)
    scatter_sequences(shape, seqs, layout, seed, kc, vc, fp8, k_scale, v_scale)
    q, cu = queries(shape, seqs, seed, q_lens)
    seq_lens = np.array([s.n for s in seqs], dtype=np.int32)
    out = oracle.paged_attention(bits16(q), cu, seq_lens, kc, vc, layout.block_table, Hq=shape.Hq,
                                 Hkv=shape.Hkv, d=shape.d, P=shape.P, scale=shape.scale, kv_fp8=fp8,
                                 k_scale=k_scale, v_scale=v_scale, split_tokens=split_tokens,
                                 nthreads=nthreads, window=window)
    return out, q, cu, kc, vc


def brute_force(shape, seqs, seed, q_lens, scale=None, dequant=None, window=0):
    """Dense numpy fp64 causal softmax(Q K^T * scale) V on the logical rows (no pages); with
    window = w > 0 a key j is visible to position p iff p - w < j <= p."""
    scale = shape.scale if scale is None else scale
    outs = []
    g = shape.Hq // shape.Hkv
    for s, ql in zip(seqs, q_lens):
        K = s.k(seed, shape).to(torch.float64).numpy()  # [n][Hkv][d]
        V = s.v(seed, shape).to(torch.float64).numpy()
        if dequant is not None:
            K, V = dequant(K, V)
        Q = s.q(seed, shape, s.n - ql, s.n).to(torch.float64).numpy()  # [ql][Hq][d]
        o = np.zeros_like(Q)
        for h in range(shape.Hq):
            kv = h // g
            sc = scale * (Q[:, h, :] @ K[:, kv, :].T)  # [ql][n]
            pos = s.n - ql + np.arange(ql)
            mask = np.arange(s.n)[None, :] <= pos[:, None]
            if window > 0:
                mask &= np.arange(s.n)[None, :] > pos[:, None] - window
            sc = np.where(mask, sc, -np.inf)
            sc = sc - sc.max(axis=1, keepdims=True)
            w = np.exp(sc)
            o[:, h, :] = (w @ V[:, kv, :]) / w.sum(axis=1, keepdims=True)
        outs.append(o)
    return np.concatenate(outs, 0)
