"""Sliding-window attention on the GPU (Vosti App. A.5: the mask adds j > p - w for a shared
window size w): parity against the fp64 oracle with the same window, and the invariance contract
-- decode equals prefill at every position, batch 1 equals batch N, chunked equals whole, page
placement does not matter -- with the window on.  A window at least as wide as the context must
give the full-attention bits."""
import numpy as np
import pytest
import torch

from synth import workloads as wl
from tests import gpu_side as gs
from tests import oracle_side as osd

pytestmark = pytest.mark.gpu

SEED = 0


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from invariant_attention_amd import binding
    binding.load()


def _eq(a, b):
    return np.array_equal(gs.bits(a), gs.bits(b))


def _setup(shape, lens, window, layout_seed=3, fp8=False, scales=(None, None)):
    seqs = wl.make_sequences(lens)
    layout = wl.layout_pages(layout_seed, lens, shape.P)
    ctx = gs.make_ctx(shape, fp8=fp8, window=window)
    pages = gs.DevicePages(shape, layout.num_pages, fp8, *scales)
    gs.fill_sequences(ctx, pages, seqs, layout, SEED)
    return seqs, layout, ctx, pages


def _check(out, ref):
    ok, err, ratio = gs.within_tolerance(out, ref)
    assert ok, f"max abs err {err}, worst err/bound {ratio}"


CASES = [
    ("tiny-w1", wl.TINY, list(wl.TINY_LENS), 1),
    ("tiny-w17", wl.TINY, list(wl.TINY_LENS), 17),
    ("tiny-w64", wl.TINY, list(wl.TINY_LENS), 64),
    ("tiny-w100", wl.TINY, list(wl.TINY_LENS), 100),
    ("tiny-w129", wl.TINY, [300, 129, 257, 64], 129),
    ("llama8b-w4096", wl.LLAMA3_8B, [8192, 4097, 4096, 2049, 700], 4096),
    ("llama8b-w2000", wl.LLAMA3_8B, [6000, 2048, 2049, 100], 2000),
    ("d64-g3-w70", wl.AttnShape(Hq=6, Hkv=2, d=64, P=16, S=64), [300, 130], 70),
]


@pytest.mark.parametrize("name,shape,lens,window", CASES, ids=[c[0] for c in CASES])
def test_window_decode_and_prefill_match_oracle(name, shape, lens, window):
    seqs, layout, ctx, pages = _setup(shape, lens, window)
    ref_d, q_d, _, _, _ = osd.run_oracle(shape, seqs, layout, SEED, [1] * len(lens), window=window)
    _check(gs.decode(ctx, pages, q_d, layout, lens), ref_d)
    q_lens = [min(n, 300) for n in lens]
    ref_p, q_p, cu, _, _ = osd.run_oracle(shape, seqs, layout, SEED, q_lens, window=window)
    _check(gs.prefill(ctx, pages, q_p, cu, layout, lens), ref_p)


def test_window_fp8_matches_oracle():
    shape = wl.LLAMA31_70B
    lens = [3000, 700]
    scales = wl.fp8_scales(4, shape.Hkv, power_of_two=False)
    seqs, layout, ctx, pages = _setup(shape, lens, 1000, fp8=True, scales=scales)
    ref, q, _, _, _ = osd.run_oracle(shape, seqs, layout, SEED, [1, 1], fp8=True, k_scale=scales[0],
                                     v_scale=scales[1], window=1000)
    _check(gs.decode(ctx, pages, q, layout, lens), ref)


@pytest.mark.parametrize("shape,lens,window", [(wl.TINY, list(wl.TINY_LENS), 37),
                                               (wl.LLAMA3_8B, [4500, 2049, 700], 1500)],
                         ids=["tiny-w37", "llama8b-w1500"])
def test_window_decode_equals_prefill_at_every_position(shape, lens, window):
    seqs, layout, ctx, pages = _setup(shape, lens, window)
    q, cu = osd.queries(shape, seqs, SEED, lens)
    pre = gs.prefill(ctx, pages, q, cu, layout, lens)
    for b, (s, n) in enumerate(zip(seqs, lens)):
        positions = sorted(set([0, 1, window - 1, window, window + 1, n - 1, n // 2]
                               + list(range(max(0, n - 70), n, 9))
                               + [p for p in (63, 64, 2047, 2048, 2049) if p < n]))
        positions = [p for p in positions if 0 <= p < n]
        qd = torch.cat([s.q(SEED, shape, p, p + 1) for p in positions])
        sub = wl.PageLayout(layout.num_pages, layout.block_table[[b] * len(positions)], [layout.pages[b]] * len(positions))
        dec = gs.decode(ctx, pages, qd, sub, [p + 1 for p in positions])
        rows = [int(cu[b]) + p for p in positions]
        assert _eq(dec, pre[rows])


def test_window_batch_and_chunk_invariance():
    shape = wl.QWEN3_8B
    window = 1024
    lens = [4096, 3000, 2500, 700]
    seqs, layout, ctx, pages = _setup(shape, lens, window)
    q, _ = osd.queries(shape, seqs, SEED, [1] * 4)
    full = gs.decode(ctx, pages, q, layout, lens)
    for b in range(4):
        one = wl.PageLayout(layout.num_pages, layout.block_table[[b]], [layout.pages[b]])
        assert _eq(gs.decode(ctx, pages, q[b:b + 1], one, [lens[b]]), full[b:b + 1])
    lay2 = wl.shuffled(layout, 4)
    pages2 = gs.DevicePages(shape, lay2.num_pages)
    gs.fill_sequences(ctx, pages2, seqs, lay2, SEED)
    assert _eq(gs.decode(ctx, pages2, q, lay2, lens), full)
    s = seqs[0]
    one = wl.PageLayout(layout.num_pages, layout.block_table[[0]], [layout.pages[0]])
    whole = gs.prefill(ctx, pages, s.q(SEED, shape, 0, 4096), np.array([0, 4096]), one, [4096])
    for budget in (64, 256, 1000):
        parts = []
        for c0 in range(0, 4096, budget):
            c1 = min(4096, c0 + budget)
            parts.append(gs.prefill(ctx, pages, s.q(SEED, shape, c0, c1), np.array([0, c1 - c0]), one, [c1]))
        assert _eq(torch.cat(parts), whole)


def test_window_wider_than_context_equals_full_attention():
    shape = wl.LLAMA3_8B
    lens = [3000, 5000, 64]
    seqs, layout, ctx_full, pages = _setup(shape, lens, 0)
    ctx_w = gs.make_ctx(shape, window=5000)
    q, cu = osd.queries(shape, seqs, SEED, [1] * 3)
    assert _eq(gs.decode(ctx_w, pages, q, layout, lens), gs.decode(ctx_full, pages, q, layout, lens))
    qp, cup = osd.queries(shape, seqs, SEED, [300, 300, 64])
    assert _eq(gs.prefill(ctx_w, pages, qp, cup, layout, lens), gs.prefill(ctx_full, pages, qp, cup, layout, lens))
