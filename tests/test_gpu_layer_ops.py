"""GPU parity and batch invariance of the layer operators through the C ABI: RMSNorm and the
fixed-tile GEMM against the fp64 oracle (|err| <= 2e-3 + 1e-2 |ref|), and a row's bits computed
alone against the same row inside larger batches at every position of a tile ("Batch invariance:
fixed splits"; Vosti, Figure 3: the matmul contract compares row x of an M-row call with row 0 of
a 1-row call)."""
import numpy as np
import pytest
import torch

from invariant_attention_amd import binding as ia
from oracle import layer_ops as lo
from synth import layer_inputs as li
from tests import gpu_side as gs

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ia.load()


def _rmsnorm(x, w, eps):
    out = torch.empty_like(x)
    ia.ia_rmsnorm(x, w, eps, out)
    torch.cuda.synchronize()
    return out.cpu()


def _gemm(a, w):
    out = torch.empty((a.shape[0], w.shape[0]), dtype=torch.bfloat16, device=DEV)
    ia.ia_gemm_bf16(a, w, out)
    torch.cuda.synchronize()
    return out.cpu()


def _bits(t):
    return t.contiguous().view(torch.int16).numpy()


@pytest.mark.parametrize("M,H,eps", [(1, 8, 1e-5), (7, 4096, 1e-5), (300, 4096, 1e-6), (5, 16384, 1e-5),
                                     (33, 136, 0.0), (2, 5120, 1e-5)])
def test_rmsnorm_matches_oracle(M, H, eps):
    x = li.activations(1, 0, M, H, scale=3.0)
    w = li.norm_weight(1, H)
    out = _rmsnorm(x.to(DEV), w.to(DEV), eps)
    ok, err, ratio = gs.within_tolerance(out, lo.rmsnorm(x, w, eps))
    assert ok, f"max abs err {err}, worst err/bound {ratio}"


def test_rmsnorm_row_alone_equals_row_in_batch():
    H = 4096
    x = li.activations(2, 0, 1000, H)
    w = li.norm_weight(2, H).to(DEV)
    full = _rmsnorm(x.to(DEV), w, 1e-5)
    for r in (0, 1, 255, 256, 999):
        one = _rmsnorm(li.activations(2, r, r + 1, H).to(DEV), w, 1e-5)
        assert np.array_equal(_bits(one), _bits(full[r:r + 1]))


@pytest.mark.parametrize("M,N,K", [(1, 256, 32), (3, 256, 64), (7, 256, 128), (300, 512, 4096),
                                   (257, 1024, 1024), (256, 256, 14336), (513, 6144, 4096),
                                   (3000, 6144, 256), (4096, 4096, 1056)])
def test_gemm_matches_oracle(M, N, K):
    a = li.activations(3, 0, M, K)
    w = li.gemm_weight(3, N, K)
    out = _gemm(a.to(DEV), w.to(DEV))
    rows = np.unique(np.linspace(0, M - 1, min(M, 64)).astype(int))  # sampled rows of the larger calls
    ref = lo.gemm(a[rows], w)
    ok, err, ratio = gs.within_tolerance(out[rows], ref)
    assert ok, f"max abs err {err}, worst err/bound {ratio}"


@pytest.mark.parametrize("N,K,Ms", [(256, 1024, (300, 1000)), (6144, 4096, (300, 4096)), (4096, 14336, (4096,)),
                                    (256, 160, (5, 700)), (4096, 1056, (4096,))])
def test_gemm_row_alone_equals_row_in_batch(N, K, Ms):
    # Rows at every position class of a tile (first, last, both halves of a 32-row MFMA block, a
    # ragged last tile), computed alone and inside larger batches.  A lone row runs on the small
    # 64 x 64 tile (K steps of 128 when K allows, else 32); the 4096-row calls at N = 6144 and
    # N = 4096 run on the 256 x 256 tile (K steps of 64, or 32 at K = 1056).
    w = li.gemm_weight(4, N, K).to(DEV)
    for M in Ms:
        a = li.activations(4, 0, M, K)
        full = _gemm(a.to(DEV), w)
        for r in sorted(r for r in {0, 1, 3, 4, 7, 8, 31, 32, 127, 128, 255, 256, 257, M - 1} if r < M):
            one = _gemm(li.activations(4, r, r + 1, K).to(DEV), w)
            assert np.array_equal(_bits(one), _bits(full[r:r + 1])), (M, r)


def test_gemm_row_bits_do_not_depend_on_its_neighbours():
    # The same row placed among different neighbours at different slots gives the same bits.
    K, N = 512, 512
    w = li.gemm_weight(5, N, K).to(DEV)
    probe = li.activations(5, 0, 1, K)
    ref = None
    for M, slot in ((1, 0), (40, 17), (260, 255), (600, 300)):
        a = li.activations(6 + M, 0, M, K).clone()
        a[slot] = probe[0]
        got = _gemm(a.to(DEV), w)[slot:slot + 1]
        ref = got if ref is None else ref
        assert np.array_equal(_bits(got), _bits(ref)), (M, slot)
