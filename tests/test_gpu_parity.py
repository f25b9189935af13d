"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded inputs.

Bar: kv_append pages bit-exact; attention outputs element-wise within |err| <= 2e-3 + 1e-2 |ref|
(bf16 inputs, fp32 accumulation, bf16 output)."""
import numpy as np
import pytest
import torch

from oracle import oracle
from synth import workloads as wl
from tests import gpu_side as gs
from tests import oracle_side as osd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from invariant_attention_amd import binding
    binding.load()  # fails loudly if the library is missing


def _setup(shape, lens, seed=0, layout_seed=3, fp8=False, scales=None, width=None, shared_prefix=0,
           by_count=False):
    seqs = wl.make_sequences(lens, shared_prefix=shared_prefix)
    layout = wl.layout_pages(layout_seed, lens, shape.P, width=width, shared_prefix=shared_prefix)
    ks, vs = scales if scales is not None else (None, None)
    ctx = gs.make_ctx(shape, fp8=fp8, by_count=by_count)
    pages = gs.DevicePages(shape, layout.num_pages, fp8, ks, vs)
    gs.fill_sequences(ctx, pages, seqs, layout, seed)
    return seqs, layout, ctx, pages


def _oracle(shape, seqs, layout, seed, q_lens, fp8=False, scales=None):
    ks, vs = scales if scales is not None else (None, None)
    out, q, cu, kc, vc = osd.run_oracle(shape, seqs, layout, seed, q_lens, fp8=fp8, k_scale=ks, v_scale=vs)
    return out, q, cu, kc, vc


# ---------------------------------------------------------------- kv_append

@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("shape", [wl.TINY, wl.LLAMA3_8B], ids=["tiny", "llama8b"])
def test_kv_append_pages_bit_exact(shape, fp8):
    rng = np.random.default_rng(1)
    num_pages = 40
    T = 300
    slots = rng.permutation(num_pages * shape.P)[:T].astype(np.int64)
    slots[::37] = -1  # padding rows are skipped
    k = wl.to_bf16(rng.standard_normal((T, shape.Hkv, shape.d)) * 3)
    v = wl.to_bf16(rng.standard_normal((T, shape.Hkv, shape.d)) * 3)
    scales = wl.fp8_scales(2, shape.Hkv, power_of_two=False) if fp8 else (None, None)
    ctx = gs.make_ctx(shape, fp8=fp8)
    pages = gs.DevicePages(shape, num_pages, fp8, *scales)
    pages.append(ctx, k, v, slots)
    torch.cuda.synchronize()
    kc, vc = osd.host_pools(shape, num_pages, fp8)
    oracle.kv_append(osd.bits16(k), osd.bits16(v), slots, kc, vc, Hkv=shape.Hkv, d=shape.d, P=shape.P,
                     kv_fp8=fp8, k_scale=scales[0], v_scale=scales[1])
    gk, gv = pages.host_bits()
    assert np.array_equal(gk, kc) and np.array_equal(gv, vc)



@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("shape", [wl.TINY, wl.LLAMA3_8B], ids=["tiny", "llama8b"])
def test_kv_append_whole_page_groups_bit_exact(shape, fp8):
    """Groups of 16 rows that fill one page in order take the transposed path; a run that starts
    mid-page, a group with a padding row, a group whose slots skip a token and a ragged tail take
    the per-row path.  Every page byte must equal the oracle's scatter."""
    rng = np.random.default_rng(2)
    num_pages = 64
    P = shape.P
    pages = rng.permutation(num_pages)
    runs = [np.arange(pages[i] * P, pages[i] * P + P) for i in range(6)]          # whole pages in order
    runs.append(np.arange(pages[6] * P + 3, pages[6] * P + P))                      # starts mid-page
    grp = np.arange(pages[7] * P, pages[7] * P + P).copy()
    grp[5] = -1                                                                     # a padding row
    runs.append(grp)
    skip = np.arange(pages[8] * P, pages[8] * P + P).copy()
    skip[9] = pages[9] * P                                                          # one token elsewhere
    runs.append(skip)
    runs.append(np.arange(pages[10] * P, pages[10] * P + 16))                       # another whole page
    runs.append(np.arange(pages[11] * P, pages[11] * P + 7))                        # ragged tail
    slots = np.concatenate(runs).astype(np.int64)
    T = len(slots)
    k = wl.to_bf16(rng.standard_normal((T, shape.Hkv, shape.d)) * 3)
    v = wl.to_bf16(rng.standard_normal((T, shape.Hkv, shape.d)) * 3)
    scales = wl.fp8_scales(2, shape.Hkv, power_of_two=False) if fp8 else (None, None)
    ctx = gs.make_ctx(shape, fp8=fp8)
    dev = gs.DevicePages(shape, num_pages, fp8, *scales)
    dev.append(ctx, k, v, slots)
    torch.cuda.synchronize()
    kc, vc = osd.host_pools(shape, num_pages, fp8)
    oracle.kv_append(osd.bits16(k), osd.bits16(v), slots, kc, vc, Hkv=shape.Hkv, d=shape.d, P=shape.P,
                     kv_fp8=fp8, k_scale=scales[0], v_scale=scales[1])
    gk, gv = dev.host_bits()
    assert np.array_equal(gk, kc) and np.array_equal(gv, vc)


# ------------------------------------------------------------------- decode

DECODE_CASES = [
    ("tiny", wl.TINY, list(wl.TINY_LENS)),
    ("tiny-edges", wl.TINY, [1, 64, 128, 129, 256, 257, 63, 2]),
    ("llama8b-B8", wl.LLAMA3_8B, wl.uniform_lens(1, 8, 512, 8192)),
    ("llama8b-edges", wl.LLAMA3_8B, [1, 2047, 2048, 2049, 4096, 4160, 8192, 65]),
    ("qwen235b-B2", wl.QWEN3_235B, [32768, 5000]),
    ("llama70b-B3", wl.LLAMA31_70B, [300, 2100, 7000]),
    ("d64-g1", wl.AttnShape(Hq=4, Hkv=4, d=64, P=16, S=192), [500, 77, 1000]),
    ("d128-g16", wl.AttnShape(Hq=16, Hkv=1, d=128, P=16, S=256), [900, 31]),
    ("d64-g3", wl.AttnShape(Hq=6, Hkv=2, d=64, P=16, S=64), [130, 64]),
]


@pytest.mark.parametrize("name,shape,lens", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_matches_oracle(name, shape, lens):
    seqs, layout, ctx, pages = _setup(shape, lens)
    ref, q, cu, _, _ = _oracle(shape, seqs, layout, 0, [1] * len(lens))
    out = gs.decode(ctx, pages, q, layout, lens)
    ok, err, ratio = gs.within_tolerance(out, ref)
    assert ok, f"max abs err {err}, worst err/bound {ratio}"


@pytest.mark.parametrize("pow2", [True, False], ids=["pow2-scales", "free-scales"])
def test_fp8_decode_matches_oracle(pow2):
    shape = wl.LLAMA31_70B
    lens = [700, 2049, 40]
    scales = wl.fp8_scales(3, shape.Hkv, pow2)
    seqs, layout, ctx, pages = _setup(shape, lens, fp8=True, scales=scales)
    ref, q, *_ = _oracle(shape, seqs, layout, 0, [1] * 3, fp8=True, scales=scales)
    out = gs.decode(ctx, pages, q, layout, lens)
    ok, err, ratio = gs.within_tolerance(out, ref)
    assert ok, f"max abs err {err}, worst err/bound {ratio}"


def test_split_by_count_variant_matches_oracle():
    shape = wl.LLAMA3_8B
    lens = wl.uniform_lens(4, 5, 512, 8192)
    seqs, layout, ctx, pages = _setup(shape, lens, by_count=True)
    ref, q, *_ = _oracle(shape, seqs, layout, 0, [1] * 5)
    out = gs.decode(ctx, pages, q, layout, lens)
    ok, err, ratio = gs.within_tolerance(out, ref)
    assert ok, f"max abs err {err}, worst err/bound {ratio}"


def test_decode_position_zero_is_v0_exactly():
    shape = wl.LLAMA3_8B
    seqs, layout, ctx, pages = _setup(shape, [1, 1])
    q, _ = osd.queries(shape, seqs, 0, [1, 1])
    out = gs.decode(ctx, pages, q, layout, [1, 1])
    for b, s in enumerate(seqs):
        v0 = s.v(0, shape, 0, 1)[0]  # [Hkv][d] bf16
        want = v0.repeat_interleave(shape.g, 0)
        assert torch.equal(out[b].cpu(), want)


def test_empty_batch_is_a_noop():
    shape = wl.TINY
    seqs, layout, ctx, pages = _setup(shape, [5])
    q = torch.zeros((0, shape.Hq, shape.d), dtype=torch.bfloat16)
    out = gs.decode(ctx, pages, q, layout, np.zeros(0, np.int32), max_seq_len=5)
    assert out.shape[0] == 0


# ------------------------------------------------------------------ prefill

PREFILL_CASES = [
    ("tiny-whole", wl.TINY, list(wl.TINY_LENS), list(wl.TINY_LENS)),
    ("tiny-chunks", wl.TINY, list(wl.TINY_LENS), [17, 37, 64, 1]),
    ("llama8b-whole-2split", wl.LLAMA3_8B, [2300, 600], [2300, 600]),
    ("llama8b-chunk", wl.LLAMA3_8B, [4096, 3000], [256, 100]),
    ("qwen235b-mixed", wl.QWEN3_235B, [32768, 512, 900], [1, 512, 512]),
    ("d64-g1", wl.AttnShape(Hq=4, Hkv=4, d=64, P=16, S=128), [300, 45], [300, 45]),
    ("d64-g3", wl.AttnShape(Hq=6, Hkv=2, d=64, P=16, S=64), [130, 64], [130, 20]),
]


@pytest.mark.parametrize("name,shape,lens,q_lens", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_matches_oracle(name, shape, lens, q_lens):
    seqs, layout, ctx, pages = _setup(shape, lens)
    ref, q, cu, *_ = _oracle(shape, seqs, layout, 0, q_lens)
    out = gs.prefill(ctx, pages, q, cu, layout, lens)
    ok, err, ratio = gs.within_tolerance(out, ref)
    assert ok, f"max abs err {err}, worst err/bound {ratio}"


def test_fp8_prefill_matches_oracle():
    shape = wl.LLAMA31_70B
    lens = [2100, 300]
    scales = wl.fp8_scales(5, shape.Hkv, False)
    seqs, layout, ctx, pages = _setup(shape, lens, fp8=True, scales=scales)
    ref, q, cu, *_ = _oracle(shape, seqs, layout, 0, [200, 300], fp8=True, scales=scales)
    out = gs.prefill(ctx, pages, q, cu, layout, lens)
    ok, err, ratio = gs.within_tolerance(out, ref)
    assert ok, f"max abs err {err}, worst err/bound {ratio}"

def test_fp8_prefill_head_dim_64_ragged():
    # e4m3 pages at head_dim 64, grouped 3:1, with tiles that end inside a page block and a
    # sequence shorter than one tile
    shape = wl.AttnShape(Hq=6, Hkv=2, d=64, P=16, S=64)
    lens = [130, 64, 7]
    scales = wl.fp8_scales(11, shape.Hkv, False)
    seqs, layout, ctx, pages = _setup(shape, lens, fp8=True, scales=scales)
    ref, q, cu, *_ = _oracle(shape, seqs, layout, 0, [130, 20, 7], fp8=True, scales=scales)
    out = gs.prefill(ctx, pages, q, cu, layout, lens)
    ok, err, ratio = gs.within_tolerance(out, ref)
    assert ok, f"max abs err {err}, worst err/bound {ratio}"

# ------------------------------------------------- unwritten page slots

@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_unwritten_slots_never_reach_the_output(fp8):
    # Keys past a sequence's end read as zero values and masked scores (Vosti App. A.2,
    # zero-padded out-of-range loads): slots of the pool that no kv_append wrote may hold
    # anything, here NaN, and decode and prefill must give the same bits as on a zeroed pool.
    shape = wl.LLAMA3_8B if not fp8 else wl.LLAMA31_70B
    lens = [2300, 600, 37, 1, 65]
    q_lens = [300, 600, 37, 1, 1]
    scales = wl.fp8_scales(5, shape.Hkv, False) if fp8 else (None, None)
    seqs = wl.make_sequences(lens)
    layout = wl.layout_pages(3, lens, shape.P)
    ctx = gs.make_ctx(shape, fp8=fp8)
    outs = []
    for poison in (False, True):
        pages = gs.DevicePages(shape, layout.num_pages, fp8, *scales)
        if poison:
            for pool in (pages.k, pages.v):
                if fp8:
                    pool.fill_(0x7F)  # e4m3 NaN
                else:
                    pool.view(torch.int16).fill_(0x7FC0)  # bf16 quiet NaN
        gs.fill_sequences(ctx, pages, seqs, layout, 0)
        q, cu = osd.queries(shape, seqs, 0, q_lens)
        dq, _ = osd.queries(shape, seqs, 0, [1] * len(lens))
        outs.append((gs.prefill(ctx, pages, q, cu, layout, lens), gs.decode(ctx, pages, dq, layout, lens)))
    (p0, d0), (p1, d1) = outs
    assert np.isfinite(p1.float().cpu().numpy()).all() and np.isfinite(d1.float().cpu().numpy()).all()
    assert np.array_equal(gs.bits(p0), gs.bits(p1))
    assert np.array_equal(gs.bits(d0), gs.bits(d1))
