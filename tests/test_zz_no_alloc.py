"""ia_paged_attn_decode_noalloc (the decode entry point that allocates nothing and takes its workspace
from the library's fixed per-GPU array) against ia_paged_attn_decode with a caller workspace, through
the C ABI: the same output bits, checked on two calls in a row with the second one smaller (the
array keeps the first call's contents), for the Llama-3-8B-shaped decode at batch 256 and a
spread-kernel launch at batch 1, and within the oracle's tolerance on the tiny config.  A launch too
big for the array is rejected before anything runs."""
import numpy as np
import pytest
import torch

from invariant_attention_amd import binding as ia
from synth import workloads as wl
from tests import gpu_side as gs
from tests import oracle_side as osd

pytestmark = pytest.mark.gpu


def _world(shape, lens, seed=0, layout_seed=3):
    seqs = wl.make_sequences(lens)
    layout = wl.layout_pages(layout_seed, lens, shape.P)
    ctx = gs.make_ctx(shape)
    pages = gs.DevicePages(shape, layout.num_pages)
    gs.fill_sequences(ctx, pages, seqs, layout, seed)
    q = torch.cat([s.q(seed, shape, s.n - 1, s.n) for s in seqs]).to(gs.DEV)
    return ctx, pages, layout, q


def _noalloc(ctx, pages, layout, q, lens, rows=None):
    rows = list(range(len(lens))) if rows is None else rows
    bt = torch.as_tensor(layout.block_table[rows], device=gs.DEV).contiguous()
    sl = torch.as_tensor(np.asarray([lens[i] for i in rows], np.int32), device=gs.DEV)
    qq = q[torch.as_tensor(rows, device=gs.DEV)].contiguous()
    out = torch.empty((len(rows),) + tuple(q.shape[1:]), dtype=torch.bfloat16, device=gs.DEV)
    ia.ia_paged_attn_decode_noalloc(ctx, qq, pages.k, pages.v, bt, sl, int(max(lens[i] for i in rows)), out,
                                    pages.k_scale, pages.v_scale)
    return out


def _with_workspace(ctx, pages, layout, q, lens, rows=None):
    rows = list(range(len(lens))) if rows is None else rows
    bt = torch.as_tensor(layout.block_table[rows], device=gs.DEV).contiguous()
    qq = q[torch.as_tensor(rows, device=gs.DEV)].contiguous()
    return gs.decode(ctx, pages, qq, None, [lens[i] for i in rows], block_table=bt)


def test_noalloc_equals_workspace_decode_batch256_then_smaller():
    shape = wl.LLAMA3_8B
    lens = wl.uniform_lens(0, 256, 512, 8192)
    ctx, pages, layout, q = _world(shape, lens)
    assert ia.ia_decode_workspace_bytes(ctx, 256, max(lens)) <= ia.ia_decode_noalloc_scratch_bytes()
    first = _noalloc(ctx, pages, layout, q, lens)
    ref = _with_workspace(ctx, pages, layout, q, lens)
    torch.cuda.synchronize()
    assert np.array_equal(gs.bits(first), gs.bits(ref))
    # A smaller second call over the contents the first one left in the array.
    rows = [5, 77, 200]
    second = _noalloc(ctx, pages, layout, q, lens, rows)
    ref2 = _with_workspace(ctx, pages, layout, q, lens, rows)
    assert np.array_equal(gs.bits(second), gs.bits(ref2))
    assert np.array_equal(gs.bits(second), gs.bits(ref[torch.as_tensor(rows, device=gs.DEV)]))


def test_noalloc_spread_launch_then_smaller():
    shape = wl.LLAMA3_8B
    lens = [6631, 2049]
    ctx, pages, layout, q = _world(shape, lens, layout_seed=4)
    first = _noalloc(ctx, pages, layout, q, lens)
    assert np.array_equal(gs.bits(first), gs.bits(_with_workspace(ctx, pages, layout, q, lens)))
    second = _noalloc(ctx, pages, layout, q, lens, [1])
    assert np.array_equal(gs.bits(second), gs.bits(_with_workspace(ctx, pages, layout, q, lens, [1])))


def test_noalloc_tiny_against_oracle_twice():
    shape = wl.TINY
    lens = list(wl.TINY_LENS)
    seqs = wl.make_sequences(lens)
    layout = wl.layout_pages(3, lens, shape.P)
    ctx = gs.make_ctx(shape)
    pages = gs.DevicePages(shape, layout.num_pages)
    gs.fill_sequences(ctx, pages, seqs, layout, 0)
    ref, q, _, _, _ = osd.run_oracle(shape, seqs, layout, 0, [1] * 4)
    q = q.to(gs.DEV)
    for rows in (list(range(4)), [2]):
        out = _noalloc(ctx, pages, layout, q, lens, rows)
        ok, err, ratio = gs.within_tolerance(out, ref[rows])
        assert ok, (rows, err, ratio)
        assert np.array_equal(gs.bits(out), gs.bits(_with_workspace(ctx, pages, layout, q, lens, rows)))


def test_noalloc_rejects_a_launch_past_the_array():
    shape = wl.LLAMA31_70B
    ctx = gs.make_ctx(shape)
    B, n = 128, 131072
    need = ia.ia_decode_workspace_bytes(ctx, B, n)
    assert need > ia.ia_decode_noalloc_scratch_bytes()
    pages = gs.DevicePages(shape, 4)
    bt = torch.zeros((B, n // 16), dtype=torch.int32, device=gs.DEV)
    sl = torch.full((B,), n, dtype=torch.int32, device=gs.DEV)
    q = torch.zeros((B, shape.Hq, shape.d), dtype=torch.bfloat16, device=gs.DEV)
    out = torch.empty_like(q)
    with pytest.raises(ia.IAError) as e:
        ia.ia_paged_attn_decode_noalloc(ctx, q, pages.k, pages.v, bt, sl, n, out)
    assert e.value.status == ia.IA_ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in str(e.value)
