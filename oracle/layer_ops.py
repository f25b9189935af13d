"""fp64 CPU oracle for the batch-invariant layer operators -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this module; the product path never does, and this module imports nothing from the product
package.  It shares no code with the HIP library: the bf16 decode below is written out here.

What the operators compute (each output row depends on its own input row only, which is what the
pages ask batch-invariant kernels to preserve):

* RMSNorm -- "Deterministic inference: results independent of the batch", "Batch invariance:
  fixed splits": normalisation reduces each row in one block in a fixed order; "Defeating
  Nondeterminism in LLM Inference" (summary page, at a glance): batch-invariant RMSNorm keeps each
  batch row's reduction on a single core.  The pages name the operator without writing it out;
  the plain reading taken here is the usual one,
      y[i] = x[i] / sqrt(mean_j x[j]^2 + eps) * w[i].
* Matrix multiplication -- Vosti, Figure 3 (the matmul contract) and the handbook's "no split-K":
  C = A W^T with A [M][K] activations (one row per token) and W [N][K] weights; every output
  element is the plain sum over k of A[m][k] W[n][k].

Everything here is fp64 (bf16 inputs are exact in fp64); numpy's fp64 matmul serves as the
library primitive for the sum over k.
"""
from __future__ import annotations

import numpy as np
import torch


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64: the bf16 value is the fp32 with those 16 high bits."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # signalling NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def _f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        assert t.dtype == torch.bfloat16
        return bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return np.asarray(t, dtype=np.float64)


def rmsnorm(x, w, eps: float) -> np.ndarray:
    """y [M][H] in fp64 for x [M][H] and gain w [H] (bf16 tensors or fp64 arrays)."""
    xf, wf = _f64(x), _f64(w)
    ms = np.mean(xf * xf, axis=1, keepdims=True)
    return xf / np.sqrt(ms + eps) * wf[None, :]


def gemm(a, w) -> np.ndarray:
    """C [M][N] = A W^T in fp64 for A [M][K] and W [N][K] (bf16 tensors or fp64 arrays)."""
    return _f64(a) @ _f64(w).T
