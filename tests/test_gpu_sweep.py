"""A seeded sweep of random attention configurations, each run through every decode kernel and
through prefill, against the fp64 oracle and against each other.

Per case (head geometry, head dim, split length, sliding window, bf16 or e4m3 pages, batch and
lengths drawn from a seeded generator, edge lengths mixed in):
- decode with each kernel (AUTO, SPLIT, WIDE, SPREAD) and both cache hints matches the oracle
  within |err| <= 2e-3 + 1e-2 |ref|, and all of them give the same bits;
- chunked prefill of the last q_len positions of each sequence matches the oracle, and gives the
  same bits under each prefill grid: in-workgroup folds (each workgroup folds its rows' splits),
  the split grid for every sequence (one workgroup per split, then a merge kernel), and the
  automatic choice; also the split grid given only the workspace the folds need (it then folds);
- the prefill row of each sequence's last position has exactly the decode output's bits (a
  decode row and the prefill row at the same position run the same operations in the same order:
  Vosti §5.3, the causal contract between prefill and decode)."""
import numpy as np
import pytest
import torch

from invariant_attention_amd import binding as ia
from synth import workloads as wl
from tests import gpu_side as gs
from tests import oracle_side as osd

pytestmark = pytest.mark.gpu

N_CASES = 32
KERNELS = [ia.IA_DECODE_AUTO, ia.IA_DECODE_SPLIT, ia.IA_DECODE_WIDE, ia.IA_DECODE_SPREAD]


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ia.load()  # fails loudly if the library is missing


def draw_case(i: int):
    """Configuration of sweep case i (deterministic in i)."""
    rng = np.random.default_rng([i, 4242])
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    d = int(rng.choice([64, 128]))
    S = 64 * int(rng.integers(1, 33))                    # 64 .. 2048 keys per split
    window = int(rng.choice([0, 0, int(rng.integers(1, 2500))]))
    fp8 = bool(rng.random() < 0.3)
    B = int(rng.integers(1, 7))
    edge = [1, 2, 63, 64, 65, S - 1, S, S + 1, 2 * S + 7]
    lens = [int(rng.choice(edge)) if rng.random() < 0.4 else int(rng.integers(1, 3001)) for _ in range(B)]
    lens = [max(1, n) for n in lens]
    # Prefill rows per sequence: a chunk ending at the last position, kept small enough that the
    # fp64 oracle finishes in seconds.
    budget = 4.0e8 / (g * Hkv * d)
    q_lens = []
    for n in lens:
        q = int(rng.integers(1, min(n, 257) + 1))
        q_lens.append(q)
    while sum(q * n for q, n in zip(q_lens, lens)) > budget and max(q_lens) > 1:
        k = int(np.argmax(q_lens))
        q_lens[k] = max(1, q_lens[k] // 2)
    shape = wl.AttnShape(Hq=g * Hkv, Hkv=Hkv, d=d, P=16, S=S)
    return shape, lens, q_lens, window, fp8


def test_sweep_cases_are_valid_and_varied():
    """(Also runs on a GPU machine with the rest; the drawn cases cover both head dims, windows, fp8,
    several groups and split lengths.)"""
    cases = [draw_case(i) for i in range(N_CASES)]
    assert {c[0].d for c in cases} == {64, 128}
    assert any(c[3] > 0 for c in cases) and any(c[3] == 0 for c in cases)
    assert any(c[4] for c in cases) and any(not c[4] for c in cases)
    assert len({c[0].Hq // c[0].Hkv for c in cases}) >= 4
    for shape, lens, q_lens, _, _ in cases:
        assert shape.Hq // shape.Hkv <= 16 and shape.S % 64 == 0
        assert all(1 <= q <= n for q, n in zip(q_lens, lens))


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep_case(case):
    shape, lens, q_lens, window, fp8 = draw_case(case)
    label = f"case {case}: Hq={shape.Hq} Hkv={shape.Hkv} d={shape.d} S={shape.S} window={window} fp8={fp8} " \
            f"lens={lens} q_lens={q_lens}"
    print(label, flush=True)
    seed = 100 + case
    seqs = wl.make_sequences(lens)
    layout = wl.layout_pages(200 + case, lens, shape.P)
    ks, vs = wl.fp8_scales(300 + case, shape.Hkv, power_of_two=bool(case % 2)) if fp8 else (None, None)
    # The oracle: decode rows (the last position of each sequence) and the prefill chunk.
    ref_dec, q_dec, _, _, _ = osd.run_oracle(shape, seqs, layout, seed, [1] * len(lens), fp8=fp8, k_scale=ks,
                                             v_scale=vs, window=window)
    ref_pf, q_pf, cu_pf, _, _ = osd.run_oracle(shape, seqs, layout, seed, q_lens, fp8=fp8, k_scale=ks,
                                               v_scale=vs, window=window)
    ctx0 = gs.make_ctx(shape, fp8=fp8, window=window)
    pages = gs.DevicePages(shape, layout.num_pages, fp8, ks, vs)
    gs.fill_sequences(ctx0, pages, seqs, layout, seed)
    outs = []
    for kernel in KERNELS:
        for hint in (ia.IA_KV_HINT_STREAM, ia.IA_KV_HINT_CACHED):
            ctx = gs.make_ctx(shape, fp8=fp8, window=window, decode_kernel=kernel, kv_cache_hint=hint)
            out = gs.decode(ctx, pages, q_dec, layout, lens)
            torch.cuda.synchronize()
            ok, err, ratio = gs.within_tolerance(out, ref_dec)
            assert ok, f"{label} decode kernel {kernel} hint {hint}: max err {err:.3e} ({ratio:.2f} of the bound)"
            outs.append(gs.bits(out))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), f"{label}: decode kernels or cache hints differ in bits"
    pf = gs.prefill(ctx0, pages, q_pf, cu_pf, layout, lens)
    torch.cuda.synchronize()
    ok, err, ratio = gs.within_tolerance(pf, ref_pf)
    assert ok, f"{label} prefill: max err {err:.3e} ({ratio:.2f} of the bound)"
    if max(lens) > shape.S:
        rows = int(q_pf.shape[0]) * shape.Hq
        fold_only = (rows * shape.d * 4 + 255) // 256 * 256 + (rows * 2 * 4 + 255) // 256 * 256
        for grid, ws in ((ia.IA_PREFILL_FOLD, None), (ia.IA_PREFILL_SPLIT, None), (ia.IA_PREFILL_SPLIT, fold_only)):
            ctx_g = gs.make_ctx(shape, fp8=fp8, window=window, prefill_grid=grid)
            o = gs.prefill(ctx_g, pages, q_pf, cu_pf, layout, lens, workspace_bytes=ws)
            torch.cuda.synchronize()
            assert np.array_equal(gs.bits(o), gs.bits(pf)), f"{label}: prefill grid {grid} (workspace {ws}) differs"
    last_rows = gs.bits(pf)[np.asarray(cu_pf[1:]) - 1]
    assert np.array_equal(last_rows, outs[0]), f"{label}: prefill's last rows differ from decode in bits"


@pytest.mark.parametrize("fp8,window", [(False, 0), (True, 0), (False, 300), (True, 300)])
def test_prefill_grids_with_empty_short_and_long_sequences(fp8, window):
    """One prefill call mixing sequences that the automatic grid splits (long keys, at most 4 row
    blocks), sequences with no rows, sequences within one split, and a long sequence of more row
    blocks (split only under IA_PREFILL_SPLIT): the three grids give the same bits, and the rows
    match the oracle."""
    shape = wl.AttnShape(Hq=16, Hkv=4, d=64, P=16, S=256)
    lens = [1500, 90, 700, 2000, 256, 257, 3000, 40]
    q_lens = [3, 0, 16, 200, 1, 257, 0, 40]
    label = f"fp8={fp8} window={window}"
    print(label, flush=True)
    seqs = wl.make_sequences(lens)
    layout = wl.layout_pages(91, lens, shape.P)
    ks, vs = wl.fp8_scales(92, shape.Hkv, power_of_two=False) if fp8 else (None, None)
    ref, q, cu, _, _ = osd.run_oracle(shape, seqs, layout, 93, q_lens, fp8=fp8, k_scale=ks, v_scale=vs,
                                      window=window)
    ctx0 = gs.make_ctx(shape, fp8=fp8, window=window)
    pages = gs.DevicePages(shape, layout.num_pages, fp8, ks, vs)
    gs.fill_sequences(ctx0, pages, seqs, layout, 93)
    outs = []
    for grid in (ia.IA_PREFILL_AUTO, ia.IA_PREFILL_FOLD, ia.IA_PREFILL_SPLIT):
        ctx = gs.make_ctx(shape, fp8=fp8, window=window, prefill_grid=grid)
        out = gs.prefill(ctx, pages, q, cu, layout, lens)
        torch.cuda.synchronize()
        ok, err, ratio = gs.within_tolerance(out, ref)
        assert ok, f"{label} grid {grid}: max err {err:.3e} ({ratio:.2f} of the bound)"
        outs.append(gs.bits(out))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), f"{label}: prefill grids differ in bits"
