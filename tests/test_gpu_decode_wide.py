"""The decode kernels are bitwise equivalent (dispatch among bitwise-equivalent kernels: Vosti,
Discussion, "Cross-kernel relational verification").  The wide kernel forms the scores and weights
of 8 tiles of a split at once and keeps only the z and value updates as a chain; the spread kernels
scores every tile of a split in its own wave and runs the chain of each 16-dim block in its own
wave.  Every row must get the same bits from each as from the split kernel, on every head geometry,
dtype, window, split policy and edge length, and the automatic choice must not change a bit either.
Both are also checked against the fp64 oracle directly."""
import numpy as np
import pytest
import torch

from invariant_attention_amd import binding as ia
from synth import workloads as wl
from tests import gpu_side as gs
from tests import oracle_side as osd

pytestmark = pytest.mark.gpu

SEED = 0


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ia.load()


def _world(shape, lens, fp8=False, scales=(None, None), layout_seed=3):
    seqs = wl.make_sequences(lens)
    layout = wl.layout_pages(layout_seed, lens, shape.P)
    ctx = gs.make_ctx(shape, fp8=fp8)
    pages = gs.DevicePages(shape, layout.num_pages, fp8, *scales)
    gs.fill_sequences(ctx, pages, seqs, layout, SEED)
    q, _ = osd.queries(shape, seqs, SEED, [1] * len(lens))
    return seqs, layout, pages, q


def _eq(a, b):
    return np.array_equal(gs.bits(a), gs.bits(b))


def _decode(shape, pages, q, layout, lens, kernel, **kw):
    ctx = gs.make_ctx(shape, fp8=pages.fp8, decode_kernel=kernel, **kw)
    return gs.decode(ctx, pages, q, layout, lens)


EDGE = [1, 2, 63, 64, 65, 127, 128, 129, 191, 300, 513, 1000]
CASES = [
    ("tiny", wl.TINY, list(wl.TINY_LENS)),
    ("tiny-edges", wl.TINY, EDGE),
    ("llama8b-B8", wl.LLAMA3_8B, wl.uniform_lens(21, 8, 512, 8192)),
    ("llama8b-edges", wl.LLAMA3_8B, [1, 2, 64, 2047, 2048, 2049, 4113, 8192, 16384 + 5]),
    ("qwen235b-g16", wl.QWEN3_235B, [32768, 5000, 17]),
    ("d64-g1", wl.AttnShape(Hq=4, Hkv=4, d=64, P=16, S=128), [300, 45, 1, 640]),
    ("d64-g3", wl.AttnShape(Hq=6, Hkv=2, d=64, P=16, S=64), [130, 64, 65, 1]),
    ("d128-g2-S64", wl.AttnShape(Hq=4, Hkv=2, d=128, P=16, S=64), [700, 63, 64, 129]),
]


KERNELS = [ia.IA_DECODE_WIDE, ia.IA_DECODE_SPREAD]
KIDS = ["wide", "spread"]


@pytest.mark.parametrize("kernel", KERNELS, ids=KIDS)
@pytest.mark.parametrize("name,shape,lens", CASES, ids=[c[0] for c in CASES])
def test_kernel_equals_split_bitwise(name, shape, lens, kernel):
    seqs, layout, pages, q = _world(shape, lens)
    split = _decode(shape, pages, q, layout, lens, ia.IA_DECODE_SPLIT)
    other = _decode(shape, pages, q, layout, lens, kernel)
    assert _eq(other, split)


@pytest.mark.parametrize("kernel", KERNELS, ids=KIDS)
@pytest.mark.parametrize("pow2", [True, False], ids=["pow2-scales", "free-scales"])
def test_kernel_equals_split_fp8(pow2, kernel):
    shape = wl.LLAMA31_70B
    lens = [3000, 700, 64, 1]
    scales = wl.fp8_scales(4, shape.Hkv, power_of_two=pow2)
    seqs, layout, pages, q = _world(shape, lens, fp8=True, scales=scales)
    split = _decode(shape, pages, q, layout, lens, ia.IA_DECODE_SPLIT)
    other = _decode(shape, pages, q, layout, lens, kernel)
    assert _eq(other, split)


@pytest.mark.parametrize("kernel", KERNELS, ids=KIDS)
@pytest.mark.parametrize("shape,lens,window", [(wl.TINY, EDGE, 17), (wl.TINY, list(wl.TINY_LENS), 100),
                                               (wl.LLAMA3_8B, [6000, 2048, 2049, 100, 4097], 2000),
                                               (wl.LLAMA3_8B, [9000, 4096], 4096)],
                         ids=["tiny-w17", "tiny-w100", "llama8b-w2000", "llama8b-w4096"])
def test_kernel_equals_split_with_window(shape, lens, window, kernel):
    seqs, layout, pages, q = _world(shape, lens)
    split = _decode(shape, pages, q, layout, lens, ia.IA_DECODE_SPLIT, window=window)
    other = _decode(shape, pages, q, layout, lens, kernel, window=window)
    assert _eq(other, split)


def test_wide_falls_back_for_long_splits():
    # A split longer than the wide kernel's 16384-key table runs on the split kernel: same bits.
    shape = wl.AttnShape(Hq=8, Hkv=2, d=64, P=16, S=32768)
    lens = [40000, 100]
    seqs, layout, pages, q = _world(shape, lens)
    split = _decode(shape, pages, q, layout, lens, ia.IA_DECODE_SPLIT)
    wide = _decode(shape, pages, q, layout, lens, ia.IA_DECODE_WIDE)
    assert _eq(wide, split)


@pytest.mark.parametrize("kernel", KERNELS, ids=KIDS)
def test_kernel_equals_split_under_split_by_count(kernel):
    shape = wl.LLAMA3_8B
    lens = [8192, 3000, 65]
    seqs, layout, pages, q = _world(shape, lens)
    split = _decode(shape, pages, q, layout, lens, ia.IA_DECODE_SPLIT, by_count=True)
    other = _decode(shape, pages, q, layout, lens, kernel, by_count=True)
    assert _eq(other, split)


@pytest.mark.parametrize("kernel", KERNELS, ids=KIDS)
@pytest.mark.parametrize("name,shape,lens", [CASES[0], CASES[3], CASES[6]], ids=["tiny", "llama8b-edges", "d64-g3"])
def test_kernel_matches_oracle(name, shape, lens, kernel):
    seqs, layout, pages, q = _world(shape, lens)
    ref, *_ = osd.run_oracle(shape, seqs, layout, SEED, [1] * len(lens))
    out = _decode(shape, pages, q, layout, lens, kernel)
    ok, err, ratio = gs.within_tolerance(out, ref)
    assert ok, f"max abs err {err}, worst err/bound {ratio}"


def test_kernel_choice_changes_no_bit_across_batch_sizes():
    # The same rows from the wide kernel alone, from the split kernel inside a large batch and
    # from the automatic choice: one set of bits.
    shape = wl.LLAMA3_8B
    lens = wl.uniform_lens(22, 64, 4096, 8192)
    seqs, layout, pages, q = _world(shape, lens)
    full_split = _decode(shape, pages, q, layout, lens, ia.IA_DECODE_SPLIT)
    full_auto = _decode(shape, pages, q, layout, lens, ia.IA_DECODE_AUTO)
    assert _eq(full_auto, full_split)
    for idx in ([0], [5, 9, 63], list(range(8))):
        sub = wl.PageLayout(layout.num_pages, layout.block_table[idx], [layout.pages[i] for i in idx])
        small = _decode(shape, pages, q[idx], sub, [lens[i] for i in idx], ia.IA_DECODE_WIDE)
        assert _eq(small, full_split[idx])


def test_spread_with_grid_bounds_above_the_lengths():
    # max_seq_len sizes the grid only.  At 4000 the spread kernels runs with most of its units and
    # tile slots empty; at 128 * 2731 its score buffer would need 2 x 3 x 2731 x 2 = 32772 slots,
    # above its 32768, and the split kernel runs instead.  Every call gives the same bits.
    shape = wl.AttnShape(Hq=8, Hkv=2, d=64, P=16, S=128)
    lens = [300, 1000, 77]
    seqs, layout, pages, q = _world(shape, lens)
    split = _decode(shape, pages, q, layout, lens, ia.IA_DECODE_SPLIT)
    ctx = gs.make_ctx(shape, decode_kernel=ia.IA_DECODE_SPREAD)
    for msl in (4000, 128 * 2731):
        wide_layout = wl.widened(layout, -(-msl // shape.P))
        bt = torch.as_tensor(wide_layout.block_table, device="cuda")
        out = gs.decode(ctx, pages, q, wide_layout, lens, max_seq_len=msl, block_table=bt)
        assert _eq(out, split), msl


def test_auto_with_a_workspace_sized_for_the_split_kernel_only():
    # Under AUTO a small launch runs the spread kernels; given only the split kernel's workspace it runs
    # the split kernel instead.  Both calls give the same bits.
    shape = wl.LLAMA3_8B
    lens = [3000, 77]  # 2 sequences x 8 kv heads x 2 splits = 32 units: AUTO's spread range
    seqs, layout, pages, q = _world(shape, lens)
    ctx = gs.make_ctx(shape)
    full = gs.decode(ctx, pages, q, layout, lens)
    split_ctx = gs.make_ctx(shape, decode_kernel=ia.IA_DECODE_SPLIT)
    need_split = ia.ia_decode_workspace_bytes(split_ctx, len(lens), max(lens))
    need_auto = ia.ia_decode_workspace_bytes(ctx, len(lens), max(lens))
    assert need_auto > need_split
    ws = torch.empty(need_split, dtype=torch.uint8, device="cuda")
    small = gs.decode(ctx, pages, q, layout, lens, ws=ws)
    assert _eq(small, full)
