"""GPU bitwise invariance: a (sequence, position) output row must have the same bits however the
work is batched, chunked, laid out in pages, reused from a prefix, or computed by decode vs
prefill (Vosti, App. A.1 contracts; Detent §8.1 invariance battery: reruns, co-batch changes,
row moves, cache splits).  Comparisons are GPU vs GPU; one pair = one (sequence, position) row
over all heads.  The split-by-count variant is the positive control: it must break batch
invariance while still matching the oracle."""
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
    from invariant_attention_amd import binding
    binding.load()


class World:
    """A set of sequences resident in one device page pool under one layout."""

    def __init__(self, shape, lens, layout_seed=3, width=None, fp8=False, scales=None, by_count=False,
                 shared_prefix=0, first_sid=0, upto=None):
        self.shape = shape
        self.lens = list(lens)
        self.seqs = wl.make_sequences(self.lens, shared_prefix=shared_prefix, first_sid=first_sid)
        self.layout = wl.layout_pages(layout_seed, self.lens, shape.P, width=width, shared_prefix=shared_prefix)
        ks, vs = scales if scales is not None else (None, None)
        self.ctx = gs.make_ctx(shape, fp8=fp8, by_count=by_count)
        self.pages = gs.DevicePages(shape, self.layout.num_pages, fp8, ks, vs)
        gs.fill_sequences(self.ctx, self.pages, self.seqs, self.layout, SEED, upto=upto)

    def with_layout(self, layout):
        w = object.__new__(World)
        w.__dict__.update(self.__dict__)
        w.layout = layout
        w.pages = gs.DevicePages(self.shape, layout.num_pages, self.pages.fp8,
                                 None if self.pages.k_scale is None else self.pages.k_scale.cpu(),
                                 None if self.pages.v_scale is None else self.pages.v_scale.cpu())
        gs.fill_sequences(w.ctx, w.pages, w.seqs, layout, SEED)
        return w

    def decode_rows(self, idx=None, pos=None, max_seq_len=None):
        """Decode output for sequences idx (default all) at positions pos (default last)."""
        idx = list(range(len(self.seqs))) if idx is None else list(idx)
        pos = [self.seqs[b].n - 1 for b in idx] if pos is None else list(pos)
        qs = torch.cat([self.seqs[b].q(SEED, self.shape, p, p + 1) for b, p in zip(idx, pos)], 0)
        sub = wl.PageLayout(self.layout.num_pages, self.layout.block_table[idx], [self.layout.pages[b] for b in idx])
        lens = [p + 1 for p in pos]
        return gs.decode(self.ctx, self.pages, qs, sub, lens, max_seq_len=max_seq_len)

    def prefill_rows(self, idx, q_lens, seq_lens=None):
        seq_lens = [self.seqs[b].n for b in idx] if seq_lens is None else list(seq_lens)
        qs = torch.cat([self.seqs[b].q(SEED, self.shape, n - ql, n) for b, ql, n in zip(idx, q_lens, seq_lens)], 0)
        cu = np.zeros(len(idx) + 1, np.int32)
        cu[1:] = np.cumsum(q_lens)
        sub = wl.PageLayout(self.layout.num_pages, self.layout.block_table[list(idx)],
                            [self.layout.pages[b] for b in idx])
        return gs.prefill(self.ctx, self.pages, qs, cu, sub, seq_lens)


def _eq(a, b):
    return np.array_equal(gs.bits(a), gs.bits(b))


def _rows_equal(a, b):
    """Per-row bit equality over all heads: returns a bool per row."""
    return [np.array_equal(x, y) for x, y in zip(gs.bits(a), gs.bits(b))]


# ----------------------------------------------------------- V1 / V7 / V8

def test_v1_tiny_batch1_vs_batch4():
    w = World(wl.TINY, wl.TINY_LENS)
    full = w.decode_rows()
    for b in range(4):
        assert _eq(w.decode_rows([b]), full[b:b + 1])


def test_v1_llama8b_batch_sizes_and_row_moves():
    lens = wl.uniform_lens(11, 64, 512, 8192)
    w = World(wl.LLAMA3_8B, lens)
    full = w.decode_rows()
    probes = [0, 7, 33, 63]
    for b in probes:
        assert _eq(w.decode_rows([b]), full[b:b + 1])
    sub8 = list(range(8))
    assert _eq(w.decode_rows(sub8), full[:8])
    rev = list(reversed(range(64)))
    assert _eq(w.decode_rows(rev), full[rev])


def test_v7_rerun():
    w = World(wl.LLAMA3_8B, wl.uniform_lens(12, 16, 512, 8192))
    a = w.decode_rows()
    b = w.decode_rows()
    assert _eq(a, b)


@pytest.mark.parametrize("neighbours", ["short", "long", "mixed"])
def test_v8_neighbours(neighbours):
    rng = np.random.default_rng(7)
    probe = 3000
    for count in (1, 4, 32):
        if neighbours == "short":
            others = list(rng.integers(1, 100, count))
        elif neighbours == "long":
            others = list(rng.integers(4000, 8193, count))
        else:
            others = list(rng.integers(1, 8193, count))
        lens = [probe] + [int(x) for x in others]
        w = World(wl.LLAMA3_8B, lens)
        alone = w.decode_rows([0])
        full = w.decode_rows()
        assert _eq(full[0:1], alone)
        moved = list(range(1, len(lens))) + [0]
        assert _eq(w.decode_rows(moved)[-1:], alone)


# ---------------------------------------------------------------- V2 / V10

def test_v2_shuffled_pages_and_table_width():
    shape = wl.LLAMA3_8B
    lens = wl.uniform_lens(13, 8, 512, 8192)
    w = World(shape, lens, width=512)
    base = w.decode_rows()
    for s in (1, 2, 3):
        w2 = w.with_layout(wl.shuffled(w.layout, s))
        assert _eq(w2.decode_rows(), base)
    w3 = w.with_layout(wl.widened(w.layout, 8192))
    assert _eq(w3.decode_rows(), base)


def test_v10_grid_bound_does_not_change_bits():
    w = World(wl.LLAMA3_8B, wl.uniform_lens(14, 8, 512, 8192), width=2048)
    base = w.decode_rows()
    assert _eq(w.decode_rows(max_seq_len=8192), base)
    assert _eq(w.decode_rows(max_seq_len=32768), base)


def test_v10_prefill_grid_bounds_do_not_change_bits():
    # max_q_len and max_seq_len size the prefill grid only.  Raising them changes the launch's
    # plan -- rows per wave (one row block for a launch this small, two once the bound makes it
    # large), which sequences run one workgroup per split, the split states' layout -- and no bit.
    w = World(wl.LLAMA3_8B, [3000, 5000, 700, 2100], width=2048)
    idx, q_lens = [0, 1, 2, 3], [64, 1, 40, 17]
    seq_lens = [w.seqs[b].n for b in idx]
    qs = torch.cat([w.seqs[b].q(SEED, w.shape, n - ql, n) for b, ql, n in zip(idx, q_lens, seq_lens)], 0)
    cu = np.zeros(len(idx) + 1, np.int32)
    cu[1:] = np.cumsum(q_lens)
    sub = wl.PageLayout(w.layout.num_pages, w.layout.block_table[idx], [w.layout.pages[b] for b in idx])
    base = gs.prefill(w.ctx, w.pages, qs, cu, sub, seq_lens)
    for mql, msl in ((64, 5000), (300, 5000), (512, 8192), (4096, 32768)):
        out = gs.prefill(w.ctx, w.pages, qs, cu, sub, seq_lens, max_seq_len=msl, max_q_len=mql)
        assert _eq(out, base), (mql, msl)


# ------------------------------------------------------------- V5 / V9 / V3

@pytest.mark.parametrize("shape,lens", [(wl.TINY, list(wl.TINY_LENS)),
                                        (wl.LLAMA3_8B, [4096, 2049, 2048, 700])],
                         ids=["tiny", "llama8b"])
def test_v5_decode_equals_prefill_at_every_position(shape, lens):
    w = World(shape, lens)
    pre = w.prefill_rows(range(len(lens)), lens)  # whole prompts
    off = 0
    for b, n in enumerate(lens):
        positions = sorted(set([0, 1, n - 1, n // 2] + list(range(max(0, n - 70), n, 7))
                               + [p for p in (63, 64, 127, 128, 2047, 2048, 2049) if p < n]))
        dec = w.decode_rows([b] * len(positions), positions)
        assert all(_rows_equal(dec, pre[[off + p for p in positions]]))
        off += n


@pytest.mark.parametrize("shape,lens", [(wl.TINY, list(wl.TINY_LENS)), (wl.LLAMA31_70B, [2100, 300])],
                         ids=["tiny", "llama70b"])
def test_v5_fp8_decode_equals_prefill(shape, lens):
    # e4m3 pages: prefill converts them while staging, decode while loading; both must give the
    # same bits at every position checked
    w = World(shape, lens, fp8=True, scales=wl.fp8_scales(21, shape.Hkv, False))
    pre = w.prefill_rows(range(len(lens)), lens)
    off = 0
    for b, n in enumerate(lens):
        positions = sorted(set([0, n - 1, n // 2] + list(range(max(0, n - 40), n, 5))
                               + [p for p in (63, 64, 127, 128, 2047, 2048) if p < n]))
        dec = w.decode_rows([b] * len(positions), positions)
        assert all(_rows_equal(dec, pre[[off + p for p in positions]]))
        off += n


def test_v9_decode_entry_equals_prefill_entry_qlen1():
    w = World(wl.LLAMA3_8B, wl.uniform_lens(15, 12, 512, 8192))
    dec = w.decode_rows()
    pre = w.prefill_rows(range(12), [1] * 12)
    assert _eq(dec, pre)


@pytest.mark.parametrize("budget", [64, 256, 1024])
def test_v3_chunk_budgets_equal_whole_prefill(budget):
    # The Qwen3-8B-shaped chunked-prefill workload at its own size: 8 prompts of 4096 tokens,
    # processed whole and in chunks (all 8 prompts' chunk k in one call).
    shape = wl.QWEN3_8B
    n, B = 4096, 8
    w = World(shape, [n] * B)
    whole = w.prefill_rows(list(range(B)), [n] * B)
    outs = []
    for c0 in range(0, n, budget):
        c1 = min(n, c0 + budget)
        # keys beyond c1 exist in the pages but are causally masked
        outs.append(w.prefill_rows(list(range(B)), [c1 - c0] * B, seq_lens=[c1] * B))
    per = [torch.cat([o[b * len(o) // B:(b + 1) * len(o) // B] for o in outs]) for b in range(B)]
    assert _eq(torch.cat(per), whole)


# ------------------------------------------------------------ positive control

def test_split_by_count_breaks_batch_invariance():
    # Load-based split count: k = max(1, min(64, 256 // B)) pieces per sequence, so the same
    # 8192-token sequence is cut into 64 pieces alone and 16 pieces in a batch of 16.
    shape = wl.LLAMA3_8B
    lens = [8192] * 16
    w = World(shape, lens)
    assert _eq(w.decode_rows()[0:1], w.decode_rows([0]))  # fixed split: invariant
    keep = w.ctx
    w.ctx = gs.make_ctx(shape, by_count=True)
    alone_c = w.decode_rows([0])
    full_c = w.decode_rows()
    w.ctx = keep
    assert not _eq(full_c[0:1], alone_c), "split-by-count unexpectedly batch invariant"


# ------------------------------------------------- dispatch order of the units
# Large launches take their units from a longest-first list built on the device
# (at least 2048 units, at most 1024 sequences); smaller ones, larger batches and
# the wide kernel use split-major grid order.  Which workgroup runs a unit must
# never change a bit.

ORDER_SHAPE = wl.AttnShape(Hq=16, Hkv=8, d=64, P=16, S=256)


@pytest.mark.parametrize("by_count,window", [(False, 0), (False, 700), (True, 0)],
                         ids=["fixed", "fixed-window", "by-count"])
def test_ordered_dispatch_changes_no_bit(by_count, window):
    shape = ORDER_SHAPE
    lens = wl.uniform_lens(31, 300, 1, 2048)  # 300 x 8 kv heads x up to 8 splits: an ordered launch
    w = World(shape, lens, by_count=by_count)
    w.ctx = gs.make_ctx(shape, by_count=by_count, window=window)
    ordered = w.decode_rows()
    w_wide = object.__new__(World)
    w_wide.__dict__.update(w.__dict__)
    w_wide.ctx = gs.make_ctx(shape, by_count=by_count, window=window, decode_kernel=ia.IA_DECODE_WIDE)
    assert _eq(w_wide.decode_rows(), ordered)  # same splits, split-major order
    if not by_count:  # by-count splits depend on the batch size by design
        for b in (0, 7, 150, 299):  # each alone: 8 units or fewer, split-major order
            assert _eq(w.decode_rows([b]), ordered[[b]]), f"row {b}"


def test_batches_above_the_order_limit_keep_their_bits():
    shape = wl.AttnShape(Hq=4, Hkv=2, d=64, P=16, S=64)
    lens = wl.uniform_lens(32, 1100, 1, 700)  # 1100 sequences: above the order list's batch limit
    w = World(shape, lens)
    full = w.decode_rows()
    idx = list(range(0, 1100, 2))  # 550 sequences x 2 kv heads x up to 11 splits: an ordered launch
    assert _eq(w.decode_rows(idx), full[idx])
    for b in (0, 549, 1099):
        assert _eq(w.decode_rows([b]), full[[b]]), f"row {b}"


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_cache_hint_changes_no_bit(fp8):
    """ia_config.kv_cache_hint picks nontemporal or cached page loads: the same bits either way, on
    a launch the automatic rule streams (>= 512 split units) and on a small one."""
    shape = wl.LLAMA3_8B
    lens = wl.uniform_lens(41, 80, 512, 8192)  # 80 x 8 kv heads x up to 4 splits
    scales = wl.fp8_scales(2, shape.Hkv, power_of_two=False) if fp8 else None
    w = World(shape, lens, fp8=fp8, scales=scales)
    outs = {}
    for name, hint in (("auto", ia.IA_KV_HINT_AUTO), ("stream", ia.IA_KV_HINT_STREAM),
                       ("cached", ia.IA_KV_HINT_CACHED)):
        w.ctx = gs.make_ctx(shape, fp8=fp8, kv_cache_hint=hint)
        outs[name] = (w.decode_rows(), w.decode_rows([0, 5]))
    for name in ("stream", "cached"):
        assert _eq(outs[name][0], outs["auto"][0]), name
        assert _eq(outs[name][1], outs["auto"][1]), name
    assert _eq(outs["auto"][1], outs["auto"][0][[0, 5]])
