"""GPU tests at the workloads' own sizes and shapes: sampled parity against the fp64 oracle in the
launch configuration the benchmark times, and the invariance variations that need a page pool,
a mixed batch, a shared prefix or fp8 pages.

Shapes are the head geometries of the models the pages measure (Llama-3-8B, Qwen3-8B,
Qwen3-235B-A22B, Llama-3.1-70B); all values are seeded synthetic N(0,1) rows.  Invariance
comparisons are GPU against GPU, bit for bit (one pair = one output row over all heads);
parity is element-wise |gpu - oracle| <= 2e-3 + 1e-2 |oracle|."""
import numpy as np
import pytest
import torch

from invariant_attention_amd import binding as ia
from oracle import oracle
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


def _world(shape, lens, layout, fp8=False, scales=(None, None), upto=None):
    seqs = wl.make_sequences(lens)
    ctx = gs.make_ctx(shape, fp8=fp8)
    pages = gs.DevicePages(shape, layout.num_pages, fp8, *scales)
    gs.fill_sequences(ctx, pages, seqs, layout, SEED, upto=upto)
    return seqs, ctx, pages


def _oracle_rows(shape, seqs, q_lens, fp8=False, scales=(None, None)):
    """Oracle output for the given sequences (own compact page layout, own scatter)."""
    layout = wl.layout_pages(7, [s.n for s in seqs], shape.P)
    ref, *_ = osd.run_oracle(shape, seqs, layout, SEED, q_lens, fp8=fp8, k_scale=scales[0], v_scale=scales[1])
    return ref


def _check(out, ref):
    ok, err, ratio = gs.within_tolerance(out, ref)
    assert ok, f"max abs err {err}, worst err/bound {ratio}"


# ------------------------------------------------ Llama-3-8B decode, batch 256

def test_llama8b_batch256_sampled_rows_match_oracle():
    """The benchmark's headline workload and launch: 256 sequences, contexts U[512, 8192], one
    decode call; sampled rows (first, last, shortest, longest, a few inside) against the oracle."""
    shape = wl.LLAMA3_8B
    lens = wl.uniform_lens(SEED, 256, 512, 8192)
    layout = wl.layout_pages(3, lens, shape.P)
    seqs, ctx, pages = _world(shape, lens, layout)
    q, _ = osd.queries(shape, seqs, SEED, [1] * 256)
    out = gs.decode(ctx, pages, q, layout, lens)
    sample = sorted({0, 1, 37, 100, 200, 255, int(np.argmin(lens)), int(np.argmax(lens))})
    ref = _oracle_rows(shape, [seqs[i] for i in sample], [1] * len(sample))
    _check(out[sample], ref)


# ------------------------------------- Qwen3-235B shape: long decode, mixed batch

@pytest.fixture(scope="module")
def qwen_mixed():
    shape = wl.QWEN3_235B
    lens = [32768] * 16 + [512] * 4
    layout = wl.layout_pages(4, lens, shape.P)
    seqs, ctx, pages = _world(shape, lens, layout)
    return shape, lens, layout, seqs, ctx, pages


def test_qwen235b_long_decode_batch1_vs_16(qwen_mixed):
    shape, lens, layout, seqs, ctx, pages = qwen_mixed
    idx = list(range(16))
    q, _ = osd.queries(shape, seqs[:16], SEED, [1] * 16)
    sub = wl.PageLayout(layout.num_pages, layout.block_table[idx], layout.pages[:16])
    full = gs.decode(ctx, pages, q, sub, lens[:16])
    for b in (0, 7, 15):
        one = wl.PageLayout(layout.num_pages, layout.block_table[[b]], [layout.pages[b]])
        assert _eq(gs.decode(ctx, pages, q[b:b + 1], one, [lens[b]]), full[b:b + 1])
    _check(full[[0, 15]], _oracle_rows(shape, [seqs[0], seqs[15]], [1, 1]))


def test_qwen235b_mixed_batch_equals_alone(qwen_mixed):
    """16 decode rows at 32768 context co-batched with 4 fresh 512-token prompts in one prefill
    call: every row equals its own run (decode entry for the decode rows, one prefill call per
    prompt), and sampled rows match the oracle.  The call runs the decode rows one workgroup per
    split (the automatic prefill grid) and gives the bits of in-workgroup folds."""
    shape, lens, layout, seqs, ctx, pages = qwen_mixed
    q_lens = [1] * 16 + [512] * 4
    q, cu = osd.queries(shape, seqs, SEED, q_lens)
    mixed = gs.prefill(ctx, pages, q, cu, layout, lens)
    folds = gs.prefill(gs.make_ctx(shape, prefill_grid=ia.IA_PREFILL_FOLD), pages, q, cu, layout, lens)
    assert _eq(mixed, folds)
    sub = wl.PageLayout(layout.num_pages, layout.block_table[:16], layout.pages[:16])
    alone_dec = gs.decode(ctx, pages, q[:16], sub, lens[:16])
    assert _eq(mixed[:16], alone_dec)
    for j in range(4):
        b = 16 + j
        one = wl.PageLayout(layout.num_pages, layout.block_table[[b]], [layout.pages[b]])
        rows = slice(int(cu[b]), int(cu[b + 1]))
        alone = gs.prefill(ctx, pages, q[rows], np.array([0, 512]), one, [512])
        assert _eq(mixed[rows], alone)
    ref = _oracle_rows(shape, [seqs[3], seqs[17]], [1, 512])
    _check(torch.cat([mixed[3:4], mixed[int(cu[17]):int(cu[18])]]), ref)


# --------------------------- Qwen3-8B chunked prefill with a cached shared prefix

def test_qwen8b_prefix_cached_equals_recomputed():
    """Prompts of 4096 tokens sharing a 2048-token prefix, driven through the library's page pool:
    the first prompt computes everything; the others find the prefix published in the pool, attach
    its pages and compute only their suffix.  Each suffix row equals, bit for bit, the same prompt
    recomputed from scratch in a fresh pool, whole and in chunks of 256."""
    shape = wl.QWEN3_8B
    n = 4096
    seqs = wl.make_sequences([n] * 4, shared_prefix=2048)
    eng = gs.MiniEngine(shape, num_pages=4 * n // 16 + 8)
    h0, c0 = eng.begin(seqs[0])
    assert c0 == 0
    eng.prefill(seqs[0], h0, 0, n)
    cached = []
    for s in seqs[1:]:
        h, c = eng.begin(s)
        assert c == 2048, "the shared prefix must be served from the cache"
        cached.append(eng.prefill(s, h, c, n))
    for s, got in zip(seqs[1:], cached):
        cold = gs.MiniEngine(shape, num_pages=n // 16 + 4)
        h, c = cold.begin(s)
        assert c == 0
        whole = cold.prefill(s, h, 0, n)
        assert _eq(got, whole[2048:])
    s = seqs[1]
    chunky = gs.MiniEngine(shape, num_pages=n // 16 + 4)
    h, _ = chunky.begin(s)
    parts = [chunky.prefill(s, h, p, p + 256) for p in range(0, n, 256)]
    assert _eq(torch.cat(parts)[2048:], cached[0])
    ref = _oracle_rows(shape, [wl.Sequence(s.sid, n, s.content)], [16])
    _check(cached[0][-16:], ref)


def test_qwen8b_whole_prefill_8x4096_sampled_rows_match_oracle():
    """The benchmark's prefill launch itself (8 prompts of 4096 tokens, Qwen3-8B shape, one call,
    the bench's page layout): sampled rows of every prompt against the oracle -- the first rows,
    the rows around the 64-key tile edges and the 2048-key split edge (2047 / 2048 / 2049), rows in
    the middle of each split, and the last rows.  The oracle computes a row at position p from the
    prompt's first p + 1 rows (what the row sees)."""
    shape = wl.QWEN3_8B
    n, B = 4096, 8
    lens = [n] * B
    seqs = wl.make_sequences(lens, first_sid=1000)
    layout = wl.layout_pages(5, lens, shape.P)
    ctx = gs.make_ctx(shape)
    pages = gs.DevicePages(shape, layout.num_pages)
    gs.fill_sequences(ctx, pages, seqs, layout, SEED)
    q, cu = osd.queries(shape, seqs, SEED, lens)
    out = gs.prefill(ctx, pages, q, cu, layout, lens)
    positions = [0, 1, 15, 63, 64, 65, 1000, 2047, 2048, 2049, 3071, 4094, 4095]
    rows, trunc = [], []
    for b, sq in enumerate(seqs):
        for p in sorted(set(positions[b % 2::2] + [2048, 4095])):  # alternate the sample between prompts
            rows.append(b * n + p)
            trunc.append(wl.Sequence(sq.sid, p + 1, sq.content[:(p + 1 + 15) // 16]))
    ref = _oracle_rows(shape, trunc, [1] * len(trunc))
    _check(out[rows], ref)


def test_qwen8b_prefill_shuffled_pages():
    shape = wl.QWEN3_8B
    lens = [3000, 4096]
    layout = wl.layout_pages(3, lens, shape.P)
    seqs, ctx, pages = _world(shape, lens, layout)
    q, cu = osd.queries(shape, seqs, SEED, lens)
    base = gs.prefill(ctx, pages, q, cu, layout, lens)
    lay2 = wl.shuffled(layout, 5)
    pages2 = gs.DevicePages(shape, lay2.num_pages)
    gs.fill_sequences(ctx, pages2, seqs, lay2, SEED)
    assert _eq(gs.prefill(ctx, pages2, q, cu, lay2, lens), base)


# ------------------------------ Llama-3.1-70B shape: shared prefix, fp8, 128K

@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_llama70b_shared_prefix_pages_equal_private_copies(fp8):
    """16 sequences sharing a 16384-token prefix (one set of refcounted physical pages) plus
    private suffixes of 256-4096 tokens, block tables 8192 wide (131072-token capacity): decode
    rows equal, bit for bit, the same sequences with private copies of the prefix, alone and
    batched; sampled rows match the oracle."""
    shape = wl.LLAMA31_70B
    rng = np.random.default_rng([SEED, 5])
    lens = [16384 + int(x) for x in rng.integers(256, 4097, 16)]
    scales = wl.fp8_scales(6, shape.Hkv, power_of_two=False) if fp8 else (None, None)
    seqs = wl.make_sequences(lens, shared_prefix=16384)
    ctx = gs.make_ctx(shape, fp8=fp8)
    shared = wl.layout_pages(3, lens, shape.P, width=8192, shared_prefix=16384)
    private = wl.layout_pages(8, lens, shape.P, width=8192)
    pa = gs.DevicePages(shape, shared.num_pages, fp8, *scales)
    for b, s in enumerate(seqs):  # the shared pages are written once, by the first sequence
        p0 = 0 if b == 0 else 16384
        pa.append(ctx, s.k(SEED, shape, p0, s.n), s.v(SEED, shape, p0, s.n), shared.slots(b, p0, s.n, shape.P))
    pb = gs.DevicePages(shape, private.num_pages, fp8, *scales)
    gs.fill_sequences(ctx, pb, seqs, private, SEED)
    q, _ = osd.queries(shape, seqs, SEED, [1] * 16)
    out_a = gs.decode(ctx, pa, q, shared, lens)
    out_b = gs.decode(ctx, pb, q, private, lens)
    assert _eq(out_a, out_b)
    one = wl.PageLayout(shared.num_pages, shared.block_table[[5]], [shared.pages[5]])
    assert _eq(gs.decode(ctx, pa, q[5:6], one, [lens[5]]), out_a[5:6])
    ref = _oracle_rows(shape, [seqs[0], seqs[9]], [1, 1], fp8=fp8, scales=scales)
    _check(out_a[[0, 9]], ref)


def test_llama70b_decode_at_131072_context():
    """One sequence at the full 131072-token capacity: decode parity, and the last 16 positions as
    one prefill chunk equal the decode rows at those positions."""
    shape = wl.LLAMA31_70B
    n = 131072
    layout = wl.layout_pages(3, [n], shape.P, width=8192)
    seqs, ctx, pages = _world(shape, [n], layout)
    q, _ = osd.queries(shape, seqs, SEED, [1])
    out = gs.decode(ctx, pages, q, layout, [n])
    _check(out, _oracle_rows(shape, seqs, [1]))
    qc, cu = osd.queries(shape, seqs, SEED, [16])
    chunk = gs.prefill(ctx, pages, qc, cu, layout, [n])
    assert _eq(chunk[-1:], out)
    for k in (0, 7):
        p = n - 16 + k
        qd = seqs[0].q(SEED, shape, p, p + 1)
        assert _eq(gs.decode(ctx, pages, qd, layout, [p + 1]), chunk[k:k + 1])


def test_fp8_pow2_scales_equal_bf16_on_dequantised_pages():
    """With power-of-two static scales, scaling commutes with every rounding (The Integer Alibi,
    §III (iii)), so the fp8 path equals, bit for bit, the bf16 path run on pages that hold the
    dequantised values (code value x scale, exact in bf16)."""
    shape = wl.LLAMA31_70B
    lens = [700, 2049, 40]
    scales = wl.fp8_scales(3, shape.Hkv, power_of_two=True)
    layout = wl.layout_pages(3, lens, shape.P)
    seqs, ctx8, p8 = _world(shape, lens, layout, fp8=True, scales=scales)
    lut = torch.tensor([oracle.e4m3_to_f64(c) for c in range(256)], dtype=torch.float64)
    ks = torch.as_tensor(scales[0], dtype=torch.float64).view(1, -1, 1, 1, 1)
    vs = torch.as_tensor(scales[1], dtype=torch.float64).view(1, -1, 1, 1)
    deq_k = (lut[p8.k.cpu().long()] * ks).to(torch.bfloat16)
    deq_v = (lut[p8.v.cpu().long()] * vs).to(torch.bfloat16)
    assert torch.equal(deq_k.double(), lut[p8.k.cpu().long()] * ks), "dequantised K must be exact in bf16"
    assert torch.equal(deq_v.double(), lut[p8.v.cpu().long()] * vs), "dequantised V must be exact in bf16"
    ctx16 = gs.make_ctx(shape)
    p16 = gs.DevicePages(shape, layout.num_pages)
    p16.k.copy_(deq_k.to(gs.DEV))
    p16.v.copy_(deq_v.to(gs.DEV))
    q, _ = osd.queries(shape, seqs, SEED, [1] * 3)
    assert _eq(gs.decode(ctx8, p8, q, layout, lens), gs.decode(ctx16, p16, q, layout, lens))
    qp, cu = osd.queries(shape, seqs, SEED, [300, 500, 40])
    assert _eq(gs.prefill(ctx8, p8, qp, cu, layout, lens), gs.prefill(ctx16, p16, qp, cu, layout, lens))


# ------------------------------------------- Vosti Figure 2 through the engine

def test_figure2_share_retain_evict_reuse_recompute():
    """Vosti Figure 2 with 16-token pages: A and B share their first page; both finish (pages
    retained, refcount 0); A's private leaf is evicted while the shared parent, which B's leaf
    still refers to, stays; C (A's prompt again) reuses the shared page, recomputes the rest into
    fresh storage and gets A's output rows bit for bit; its generated positions (decode, evicting
    B's leaf for space) equal a cold run's."""
    from invariant_attention_amd import binding as ia
    shape = wl.TINY
    seqs = wl.make_sequences([40, 40], shared_prefix=16)
    a, b = seqs
    eng = gs.MiniEngine(shape, num_pages=3)
    ha, ca = eng.begin(a, 32)
    out_a = eng.prefill(a, ha, ca, 32)
    hb, cb = eng.begin(b, 32)
    assert (ca, cb) == (0, 16)
    eng.prefill(b, hb, cb, 32)
    shared = int(ia.ia_seq_block_table(ha)[0])
    assert int(ia.ia_seq_block_table(hb)[0]) == shared and ia.ia_pool_page_refs(eng.pool, shared) == 2
    eng.end(ha)
    eng.end(hb)
    assert ia.ia_pool_page_refs(eng.pool, shared) == 0 and ia.ia_pool_page_published(eng.pool, shared)
    assert ia.ia_pool_evict(eng.pool, 1) == 1                 # A's leaf: released first
    assert ia.ia_pool_page_published(eng.pool, shared)        # the parent stays
    hc, cc = eng.begin(a, 32)
    assert cc == 16
    out_c = eng.prefill(a, hc, cc, 32)
    assert _eq(out_c, out_a[16:])
    gen_c = torch.cat([eng.decode(a, hc, p) for p in range(32, 40)])
    cold = gs.MiniEngine(shape, num_pages=3)
    h, _ = cold.begin(a, 32)
    assert _eq(cold.prefill(a, h, 0, 32)[16:], out_c)
    assert _eq(torch.cat([cold.decode(a, h, p) for p in range(32, 40)]), gen_c)
    _check(out_a, _oracle_rows(shape, [wl.Sequence(a.sid, 32, a.content[:2].copy())], [32]))
    _check(gen_c, _oracle_rows(shape, [a], [8]))
