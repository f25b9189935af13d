"""Seeded synthetic inputs for paged attention.

This module holds no attention arithmetic.  It draws the logical K/V/Q rows
of synthetic sequences, picks their lengths, and lays them out over a shuffled
pool of physical pages (page tables and slot mappings).  Both the oracle-side
tests and the GPU-side tests and bench take their inputs from here, so the
two sides see the same bits.

Values: fp32 N(0,1) from ``numpy.random.default_rng``, rounded to bf16 by
round-to-nearest-even (torch's CPU conversion).  Rows are drawn in blocks of
16 positions from a generator keyed by (seed, content id, stream, block), so
any range of positions of any sequence can be produced on its own -- a
sampled parity check at full size only draws the sequences it samples.  A
shared prefix is the same content id for the positions it covers, so every
sequence that shares it gets bit-identical rows there (what a model would
compute for an identical token prefix).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

ROW_BLOCK = 16
_STREAM_K, _STREAM_V, _STREAM_Q = 1, 2, 3


@dataclass(frozen=True)
class AttnShape:
    Hq: int
    Hkv: int
    d: int
    P: int = 16
    S: int = 2048

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.d)))


# The workload shapes the method is measured on (head geometry of the models
# the pages test with; lengths and batch sizes per workload).
TINY = AttnShape(Hq=8, Hkv=2, d=64, P=16, S=128)
LLAMA3_8B = AttnShape(Hq=32, Hkv=8, d=128, P=16, S=2048)
QWEN3_8B = AttnShape(Hq=32, Hkv=8, d=128, P=16, S=2048)
QWEN3_235B = AttnShape(Hq=64, Hkv=4, d=128, P=16, S=2048)
LLAMA31_70B = AttnShape(Hq=64, Hkv=8, d=128, P=16, S=2048)
TINY_LENS = (17, 100, 211, 300)


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """fp32 array -> bf16 tensor by round-to-nearest-even."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _block_rows(seed: int, content: int, stream: int, blk: int, heads: int, d: int) -> np.ndarray:
    rng = np.random.default_rng([seed, content, stream, blk])
    return rng.standard_normal((ROW_BLOCK, heads, d), dtype=np.float32)


def rows(seed: int, content_ids: np.ndarray, stream: int, heads: int, d: int, p0: int, p1: int) -> torch.Tensor:
    """bf16 rows for positions [p0, p1); content_ids[p] names the generator of position p's block."""
    out = np.empty((p1 - p0, heads, d), dtype=np.float32)
    p = p0
    while p < p1:
        blk = p // ROW_BLOCK
        hi = min(p1, (blk + 1) * ROW_BLOCK)
        src = _block_rows(seed, int(content_ids[blk]), stream, blk, heads, d)
        out[p - p0:hi - p0] = src[p - blk * ROW_BLOCK:hi - blk * ROW_BLOCK]
        p = hi
    return to_bf16(out)


@dataclass
class Sequence:
    """One synthetic sequence: length n and the content id of each 16-position block."""
    sid: int
    n: int
    content: np.ndarray  # [ceil(n/16)] int64

    def k(self, seed: int, shape: AttnShape, p0: int = 0, p1: int | None = None) -> torch.Tensor:
        return rows(seed, self.content, _STREAM_K, shape.Hkv, shape.d, p0, self.n if p1 is None else p1)

    def v(self, seed: int, shape: AttnShape, p0: int = 0, p1: int | None = None) -> torch.Tensor:
        return rows(seed, self.content, _STREAM_V, shape.Hkv, shape.d, p0, self.n if p1 is None else p1)

    def q(self, seed: int, shape: AttnShape, p0: int, p1: int) -> torch.Tensor:
        return rows(seed, self.content, _STREAM_Q, shape.Hq, shape.d, p0, p1)

    def tokens(self, p0: int = 0, p1: int | None = None) -> list[int]:
        """Synthetic token ids of positions [p0, p1): a function of the position and of its block's
        content id, so sequences that share a prefix share its tokens (what a prefix cache keys on)."""
        p1 = self.n if p1 is None else p1
        pos = np.arange(p0, p1, dtype=np.int64)
        c = self.content[pos // ROW_BLOCK]
        return [int(x) for x in ((c * 1000003 + pos * 7919) % 49999 + 1)]


def make_sequences(lens, shared_prefix: int = 0, first_sid: int = 0) -> list[Sequence]:
    """Sequences with the given lengths; the first `shared_prefix` positions (a multiple of 16)
    draw from one common content id (1 << 40), so they are bit-identical across sequences."""
    assert shared_prefix % ROW_BLOCK == 0
    out = []
    for i, n in enumerate(lens):
        sid = first_sid + i
        nblk = -(-int(n) // ROW_BLOCK)
        content = np.full(nblk, sid, dtype=np.int64)
        content[:min(nblk, shared_prefix // ROW_BLOCK)] = 1 << 40
        out.append(Sequence(sid=sid, n=int(n), content=content))
    return out


def uniform_lens(seed: int, count: int, lo: int, hi: int) -> list[int]:
    """Lengths uniform in [lo, hi] (inclusive)."""
    rng = np.random.default_rng([seed, 7])
    return [int(x) for x in rng.integers(lo, hi + 1, size=count)]


@dataclass
class PageLayout:
    """Physical placement of a batch: a block table row per sequence and a pool size."""
    num_pages: int
    block_table: np.ndarray  # [B][width] int32, unused entries -1
    pages: list[np.ndarray] = field(default_factory=list)  # per sequence, its page ids in order

    def slots(self, b: int, p0: int, p1: int, P: int) -> np.ndarray:
        pos = np.arange(p0, p1, dtype=np.int64)
        return self.pages[b][pos // P].astype(np.int64) * P + pos % P


def layout_pages(seed: int, lens, P: int, width: int | None = None, shared_prefix: int = 0,
                 slack: float = 1.25, min_pages: int = 0) -> PageLayout:
    """Assign each sequence's logical pages to physical pages of a pool 1.25x the demand, in a
    seeded random order.  The first shared_prefix // P logical pages are one set of physical
    pages shared by every sequence (a refcounted prefix)."""
    lens = [int(n) for n in lens]
    n_shared = shared_prefix // P
    need = [-(-n // P) for n in lens]
    demand = n_shared + sum(max(0, k - n_shared) for k in need)
    num_pages = max(int(np.ceil(demand * slack)) + 1, min_pages, 1)
    rng = np.random.default_rng([seed, 11])
    perm = rng.permutation(num_pages).astype(np.int64)
    shared = perm[:n_shared]
    cursor = n_shared
    if width is None:
        width = max(need) if need else 1
    bt = np.full((len(lens), max(width, 1)), -1, dtype=np.int32)
    pages = []
    for b, k in enumerate(need):
        own = perm[cursor:cursor + max(0, k - n_shared)]
        cursor += max(0, k - n_shared)
        pg = np.concatenate([shared[:min(k, n_shared)], own]).astype(np.int64)
        assert len(pg) <= width, "block table too narrow"
        bt[b, :len(pg)] = pg
        pages.append(pg)
    return PageLayout(num_pages=num_pages, block_table=bt, pages=pages)


def shuffled(layout: PageLayout, seed: int) -> PageLayout:
    """The same logical batch on a different random permutation of physical pages (shared pages
    stay shared)."""
    rng = np.random.default_rng([seed, 13])
    perm = rng.permutation(layout.num_pages).astype(np.int64)
    pages = [perm[p] for p in layout.pages]
    bt = np.full_like(layout.block_table, -1)
    for b, pg in enumerate(pages):
        bt[b, :len(pg)] = pg
    return PageLayout(num_pages=layout.num_pages, block_table=bt, pages=pages)


def widened(layout: PageLayout, width: int) -> PageLayout:
    bt = np.full((layout.block_table.shape[0], width), -1, dtype=np.int32)
    for b, pg in enumerate(layout.pages):
        bt[b, :len(pg)] = pg
    return PageLayout(num_pages=layout.num_pages, block_table=bt, pages=list(layout.pages))


def fp8_scales(seed: int, Hkv: int, power_of_two: bool) -> tuple[np.ndarray, np.ndarray]:
    """Static per-KV-head fp8 scales for K and V: powers of two in [2^-6, 2^-4], or values
    drawn uniformly from [0.01, 0.05]."""
    rng = np.random.default_rng([seed, 17])
    if power_of_two:
        ks = np.exp2(rng.integers(-6, -3, size=Hkv)).astype(np.float32)
        vs = np.exp2(rng.integers(-6, -3, size=Hkv)).astype(np.float32)
    else:
        ks = rng.uniform(0.01, 0.05, size=Hkv).astype(np.float32)
        vs = rng.uniform(0.01, 0.05, size=Hkv).astype(np.float32)
    return ks, vs
