"""Seeded synthetic inputs for the batch-invariant layer operators (RMSNorm, the fixed-tile GEMM).

No operator arithmetic lives here: it only draws bf16 tensors.  Activation rows are drawn in blocks
of 16 rows from a generator keyed by (seed, stream, block), so any row range can be produced on
its own (a row computed alone and the same row inside a large batch see the same bits).  GEMM
weights are N(0, 1/K) so that outputs are O(1); the scaling happens in fp32 before the bf16
rounding, as part of drawing the input.
"""
from __future__ import annotations

import numpy as np
import torch

ROW_BLOCK = 16
_STREAM_ACT, _STREAM_W, _STREAM_NORM = 11, 12, 13


def _bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def activations(seed: int, row0: int, row1: int, K: int, scale: float = 1.0) -> torch.Tensor:
    """Rows row0..row1-1 of an activation matrix [*, K] (bf16, N(0, scale^2))."""
    out = np.empty((row1 - row0, K), np.float32)
    b0, b1 = row0 // ROW_BLOCK, (row1 + ROW_BLOCK - 1) // ROW_BLOCK
    for blk in range(b0, b1):
        rows = np.random.default_rng([seed, _STREAM_ACT, K, blk]).standard_normal((ROW_BLOCK, K), dtype=np.float32)
        lo, hi = max(row0, blk * ROW_BLOCK), min(row1, (blk + 1) * ROW_BLOCK)
        out[lo - row0:hi - row0] = rows[lo - blk * ROW_BLOCK:hi - blk * ROW_BLOCK] * np.float32(scale)
    return _bf16(out)


def gemm_weight(seed: int, N: int, K: int) -> torch.Tensor:
    """A weight matrix W [N][K] (the output features' rows, as a linear layer stores them), N(0, 1/K)."""
    w = np.random.default_rng([seed, _STREAM_W, N, K]).standard_normal((N, K), dtype=np.float32)
    return _bf16(w * np.float32(1.0 / np.sqrt(K)))


def norm_weight(seed: int, H: int) -> torch.Tensor:
    """An RMSNorm gain vector [H], around 1."""
    g = np.random.default_rng([seed, _STREAM_NORM, H]).standard_normal(H, dtype=np.float32)
    return _bf16(1.0 + 0.1 * g)
