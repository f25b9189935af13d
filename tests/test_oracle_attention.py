"""Pins for the oracle's paged attention, against things other than itself:

* dense numpy fp64 softmax on the logical rows (no pages, no gather) -- a different formulation;
* torch's scaled_dot_product_attention in fp64 on the CPU -- an independent library routine;
* closed forms: q = 0 gives the mean of v_0..v_p; two keys give a logistic weight that fixes the
  scale; a dominant key returns its value row; position 0 returns v_0 exactly;
* invariants: a permutation of physical pages leaves the output bit-identical; the fixed-split
  form (flash-decoding with an ascending LSE merge) agrees with the plain form;
* the worked example of Vosti Figure 4 (prefill row 3 of 6 vs decode at k_len 4, different
  physical pages): bit-equal outputs at the same logical position;
* fp8 pages: attention over the stored e4m3 codes equals the dense result on the dequantised rows.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import oracle
from synth import workloads as wl
from tests import oracle_side as osd
from tests import golden

SHAPES = [
    wl.AttnShape(Hq=8, Hkv=2, d=64, P=16, S=128),   # the tiny decode shape
    wl.AttnShape(Hq=4, Hkv=4, d=64, P=16, S=64),    # g = 1
    wl.AttnShape(Hq=16, Hkv=2, d=128, P=16, S=64),  # g = 8, d = 128
    wl.AttnShape(Hq=6, Hkv=3, d=32, P=2, S=64),     # tiny pages
]


def _close(a, b, rtol=1e-12):
    scale = np.maximum(np.abs(b), 1e-3)
    return np.max(np.abs(a - b) / scale)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"h{s.Hq}-{s.Hkv}-d{s.d}-P{s.P}")
@pytest.mark.parametrize("mode", ["decode", "prefill", "chunk"])
def test_oracle_matches_dense_bruteforce(oracle_lib, shape, mode):
    lens = list(wl.TINY_LENS)
    seqs = wl.make_sequences(lens)
    layout = wl.layout_pages(3, lens, shape.P)
    q_lens = {"decode": [1] * 4, "prefill": lens, "chunk": [5, 64, 33, 17]}[mode]
    out, *_ = osd.run_oracle(shape, seqs, layout, 0, q_lens)
    ref = osd.brute_force(shape, seqs, 0, q_lens)
    assert _close(out, ref) < 1e-12


def test_oracle_matches_torch_sdpa(oracle_lib):
    shape = wl.AttnShape(Hq=8, Hkv=2, d=64, P=16, S=128)
    lens = [40, 75, 130]
    q_lens = [40, 9, 1]
    seqs = wl.make_sequences(lens, first_sid=20)
    layout = wl.layout_pages(4, lens, shape.P)
    out, *_ = osd.run_oracle(shape, seqs, layout, 1, q_lens)
    refs = []
    for s, ql in zip(seqs, q_lens):
        K = s.k(1, shape).to(torch.float64).permute(1, 0, 2).repeat_interleave(shape.g, 0)  # [Hq][n][d]
        V = s.v(1, shape).to(torch.float64).permute(1, 0, 2).repeat_interleave(shape.g, 0)
        Q = s.q(1, shape, s.n - ql, s.n).to(torch.float64).permute(1, 0, 2)  # [Hq][ql][d]
        pos = torch.arange(s.n - ql, s.n)[:, None]
        mask = torch.arange(s.n)[None, :] <= pos
        o = F.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=mask[None, None],
                                           scale=shape.scale)[0]
        refs.append(o.permute(1, 0, 2).numpy())
    assert _close(out, np.concatenate(refs, 0)) < 1e-12


# ------------------------------------------------------------ closed forms

def _oracle_on_rows(shape, K, V, Q, q_len, pages=None, scale=None):
    """Oracle on explicit logical rows of one sequence: K, V [n][Hkv][d] and Q [q_len][Hq][d] bf16."""
    n = K.shape[0]
    npg = -(-n // shape.P)
    if pages is None:
        pages = np.arange(npg, dtype=np.int64)
    num_pages = int(max(pages)) + 1
    kc, vc = osd.host_pools(shape, num_pages)
    pos = np.arange(n)
    slots = pages[pos // shape.P] * shape.P + pos % shape.P
    oracle.kv_append(osd.bits16(K), osd.bits16(V), slots, kc, vc, Hkv=shape.Hkv, d=shape.d, P=shape.P)
    bt = np.asarray(pages, dtype=np.int32)[None, :]
    return oracle.paged_attention(osd.bits16(Q), np.array([0, q_len], np.int32), np.array([n], np.int32),
                                  kc, vc, bt, Hq=shape.Hq, Hkv=shape.Hkv, d=shape.d, P=shape.P,
                                  scale=shape.scale if scale is None else scale)


def _bf16(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def test_zero_query_gives_mean_of_visible_values(oracle_lib):
    shape = wl.AttnShape(Hq=2, Hkv=1, d=16, P=4, S=64)
    rng = np.random.default_rng(0)
    n = 23
    K = _bf16(rng.standard_normal((n, 1, 16)))
    V = _bf16(rng.standard_normal((n, 1, 16)))
    Q = _bf16(np.zeros((n, 2, 16)))
    out = _oracle_on_rows(shape, K, V, Q, q_len=n)
    Vd = V.to(torch.float64).numpy()[:, 0, :]
    for i in range(n):
        mean = Vd[:i + 1].mean(axis=0)
        assert np.max(np.abs(out[i, 0] - mean)) < 1e-14 and np.max(np.abs(out[i, 1] - mean)) < 1e-14


def test_two_keys_fix_the_scale(oracle_lib):
    # q = a e_0, k_0 = b e_0, k_1 = 0  ->  s_0 = scale*a*b, s_1 = 0,
    # O = (e^{s_0} v_0 + v_1) / (e^{s_0} + 1).
    shape = wl.AttnShape(Hq=1, Hkv=1, d=16, P=16, S=64)
    a, b = 3.0, 1.5
    K = np.zeros((2, 1, 16), np.float32); K[0, 0, 0] = b
    V = np.zeros((2, 1, 16), np.float32); V[0, 0, :] = 1.0; V[1, 0, :] = -2.0
    Q = np.zeros((1, 1, 16), np.float32); Q[0, 0, 0] = a
    out = _oracle_on_rows(shape, _bf16(K), _bf16(V), _bf16(Q), q_len=1)
    s0 = shape.scale * a * b
    w = np.exp(s0) / (np.exp(s0) + 1)
    assert np.max(np.abs(out[0, 0] - (w * 1.0 + (1 - w) * -2.0))) < 1e-14
    out2 = _oracle_on_rows(shape, _bf16(K), _bf16(V), _bf16(Q), q_len=1, scale=0.5)
    w2 = np.exp(0.5 * a * b) / (np.exp(0.5 * a * b) + 1)
    assert np.max(np.abs(out2[0, 0] - (w2 - 2 * (1 - w2)))) < 1e-14


def test_dominant_key_returns_its_value_row(oracle_lib):
    shape = wl.AttnShape(Hq=2, Hkv=1, d=32, P=16, S=64)
    rng = np.random.default_rng(1)
    n, jstar = 50, 17
    K = rng.standard_normal((n, 1, 32)).astype(np.float32) * 0.01
    V = rng.standard_normal((n, 1, 32)).astype(np.float32)
    q = np.zeros(32, np.float32); q[:4] = 1.0
    K[jstar, 0] = 0.0; K[jstar, 0, :4] = 256.0    # score scale*1024 dominates every other key
    Q = np.tile(q, (1, 2, 1))
    out = _oracle_on_rows(shape, _bf16(K), _bf16(V), _bf16(Q), q_len=1)
    Vd = _bf16(V).to(torch.float64).numpy()
    assert np.max(np.abs(out[0, 0] - Vd[jstar, 0])) < 1e-12


def test_position_zero_returns_v0_exactly(oracle_lib):
    shape = wl.TINY
    seqs = wl.make_sequences([1, 30])
    layout = wl.layout_pages(2, [1, 30], shape.P)
    out, *_ = osd.run_oracle(shape, seqs, layout, 0, [1, 30])
    v0 = seqs[0].v(0, shape).to(torch.float64).numpy()[0]
    for h in range(shape.Hq):
        assert np.array_equal(out[0, h], v0[h // shape.g])
    v0b = seqs[1].v(0, shape).to(torch.float64).numpy()[0]
    for h in range(shape.Hq):  # row 0 of the 30-token prefill is position 0 too
        assert np.array_equal(out[1, h], v0b[h // shape.g])


# ------------------------------------------------------------- invariants

def test_page_permutation_leaves_output_bit_identical(oracle_lib):
    shape = wl.TINY
    lens = list(wl.TINY_LENS)
    seqs = wl.make_sequences(lens)
    base = wl.layout_pages(3, lens, shape.P)
    out0, *_ = osd.run_oracle(shape, seqs, base, 0, [3, 1, 7, 1])
    for s in (1, 2, 3):
        out1, *_ = osd.run_oracle(shape, seqs, wl.shuffled(base, s), 0, [3, 1, 7, 1])
        assert np.array_equal(out0, out1)
    out2, *_ = osd.run_oracle(shape, seqs, wl.widened(base, 64), 0, [3, 1, 7, 1])
    assert np.array_equal(out0, out2)


@pytest.mark.parametrize("split", [16, 64, 128])
def test_fixed_split_merge_agrees_with_plain(oracle_lib, split):
    shape = wl.TINY
    lens = list(wl.TINY_LENS)
    seqs = wl.make_sequences(lens)
    layout = wl.layout_pages(3, lens, shape.P)
    plain, *_ = osd.run_oracle(shape, seqs, layout, 0, lens)
    split_out, *_ = osd.run_oracle(shape, seqs, layout, 0, lens, split_tokens=split)
    assert _close(split_out, plain) < 1e-12


def test_vosti_figure4_prefill_row_equals_decode(oracle_lib):
    # Vosti, Figure 4 (tests/golden/vosti_figure4_positions.txt): a prefill invocation on pages
    # P7, P9, P2 and a decode invocation on pages P4, P8 (two tokens a page) reach the same logical
    # position, and their selected rows are bitwise equal.
    fix = golden.load("vosti_figure4_positions.txt")
    pre_f, dec_f = golden.one(fix, "prefill"), golden.one(fix, "decode")
    P, pos = int(golden.one(fix, "page_size")), int(golden.one(fix, "position"))
    for f in (pre_f, dec_f):
        assert int(f["k_len"]) - int(f["q_len"]) + int(f["row"]) == pos
        assert len(golden.ints(f["pages"])) == -(-int(f["k_len"]) // P)
    shape = wl.AttnShape(Hq=2, Hkv=1, d=16, P=P, S=64)
    n_pre, n_dec = int(pre_f["k_len"]), int(dec_f["k_len"])
    rng = np.random.default_rng(4)
    K = _bf16(rng.standard_normal((n_pre, 1, 16)))
    V = _bf16(rng.standard_normal((n_pre, 1, 16)))
    Q = _bf16(rng.standard_normal((n_pre, 2, 16)))
    pre = _oracle_on_rows(shape, K, V, Q, q_len=int(pre_f["q_len"]), pages=np.array(golden.ints(pre_f["pages"])))
    q_dec = Q[pos - int(dec_f["row"]):pos - int(dec_f["row"]) + int(dec_f["q_len"])]
    dec = _oracle_on_rows(shape, K[:n_dec], V[:n_dec], q_dec, q_len=int(dec_f["q_len"]),
                          pages=np.array(golden.ints(dec_f["pages"])))
    equal = np.array_equal(pre[int(pre_f["row"])], dec[int(dec_f["row"])])
    assert equal == golden.flag(golden.one(fix, "outputs")["bitwise_equal"])
    # and a wrong position rule (p = i) would have given row 0 instead:
    assert not np.array_equal(pre[0], dec[int(dec_f["row"])])


@pytest.mark.parametrize("pow2", [True, False])
def test_fp8_pages_match_dequantised_dense(oracle_lib, pow2):
    shape = wl.AttnShape(Hq=8, Hkv=2, d=64, P=16, S=128)
    lens = [33, 90]
    seqs = wl.make_sequences(lens)
    layout = wl.layout_pages(5, lens, shape.P)
    ks, vs = wl.fp8_scales(0, shape.Hkv, pow2)
    out, *_ = osd.run_oracle(shape, seqs, layout, 0, [1, 90], fp8=True, k_scale=ks, v_scale=vs)

    def dequant(K, V):
        Kq = np.empty_like(K); Vq = np.empty_like(V)
        for h in range(shape.Hkv):
            kq = np.array([oracle.quantize_e4m3(x, ks[h]) for x in K[:, h, :].ravel()], np.uint8)
            vq = np.array([oracle.quantize_e4m3(x, vs[h]) for x in V[:, h, :].ravel()], np.uint8)
            dec = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
            Kq[:, h, :] = dec[kq].reshape(K[:, h, :].shape) * np.float64(ks[h])
            Vq[:, h, :] = dec[vq].reshape(V[:, h, :].shape) * np.float64(vs[h])
        return Kq, Vq

    ref = osd.brute_force(shape, seqs, 0, [1, 90], dequant=dequant)
    assert _close(out, ref) < 1e-12


# K slot of each token of a 16-token page: tokens 0-3, 8-11, 4-7, 12-15 fill slots 0..15, so that
# the 8 tokens one MFMA score block takes from a page (0-3 with 8-11, or 4-7 with 12-15) are 8
# consecutive 16-byte units.
K_SLOT_16 = [0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15]


def test_kv_append_layout(oracle_lib):
    """Byte placement of the page layout, read back with numpy indexing rather than index
    arithmetic: K[page][head][dim // 8][K_SLOT_16[token]][dim % 8], V[page][head][dim][token]."""
    shape = wl.AttnShape(Hq=4, Hkv=2, d=32, P=16, S=64)
    rng = np.random.default_rng(2)
    T = 40
    k = _bf16(rng.standard_normal((T, 2, 32)))
    v = _bf16(rng.standard_normal((T, 2, 32)))
    slots = rng.permutation(8 * 16)[:T].astype(np.int64)
    kc, vc = osd.host_pools(shape, 8)
    oracle.kv_append(osd.bits16(k), osd.bits16(v), slots, kc, vc, Hkv=2, d=32, P=16)
    kb, vb = osd.bits16(k), osd.bits16(v)
    for t in range(T):
        page, tok = divmod(int(slots[t]), 16)
        for h in range(2):
            assert np.array_equal(kc[page, h, :, K_SLOT_16[tok], :].reshape(-1), kb[t, h])
            assert np.array_equal(vc[page, h, :, tok], vb[t, h])
    # untouched slots stay zero
    written = np.zeros(8 * 16, bool); written[slots] = True
    for s in np.nonzero(~written)[0]:
        page, tok = divmod(int(s), 16)
        assert not kc[page, :, :, K_SLOT_16[tok], :].any() and not vc[page, :, :, tok].any()


@pytest.mark.parametrize("P", [4, 8, 32])
def test_kv_append_layout_other_page_sizes(oracle_lib, P):
    """Pages of fewer than 16 tokens keep K in token order; a 32-token page applies the 16-token
    slot order to each of its two groups of 16."""
    shape = wl.AttnShape(Hq=2, Hkv=1, d=16, P=P, S=64)
    rng = np.random.default_rng(3)
    T = 4 * P
    k = _bf16(rng.standard_normal((T, 1, 16)))
    v = _bf16(rng.standard_normal((T, 1, 16)))
    slots = np.arange(T, dtype=np.int64)
    kc, vc = osd.host_pools(shape, 4)
    oracle.kv_append(osd.bits16(k), osd.bits16(v), slots, kc, vc, Hkv=1, d=16, P=P)
    kb = osd.bits16(k)
    for t in range(T):
        page, tok = divmod(t, P)
        want = tok if P < 16 else 16 * (tok // 16) + K_SLOT_16[tok % 16]
        assert np.array_equal(kc[page, 0, :, want, :].reshape(-1), kb[t, 0])


# ------------------------------------------------------ sliding window (Vosti App. A.5)

WINDOWS = [1, 5, 16, 64, 100, 250, 1000]


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("mode", ["decode", "prefill", "chunk"])
def test_window_matches_dense_bruteforce(oracle_lib, window, mode):
    """Sliding window of w keys: position p sees keys p - w < j <= p (dense numpy fp64 on logical
    rows, a different formulation), in plain and fixed-split form."""
    shape = wl.AttnShape(Hq=8, Hkv=2, d=64, P=16, S=64)
    lens = list(wl.TINY_LENS)
    seqs = wl.make_sequences(lens)
    layout = wl.layout_pages(3, lens, shape.P)
    q_lens = {"decode": [1] * 4, "prefill": lens, "chunk": [5, 64, 33, 17]}[mode]
    ref = osd.brute_force(shape, seqs, 0, q_lens, window=window)
    for split in (0, shape.S):
        out, *_ = osd.run_oracle(shape, seqs, layout, 0, q_lens, window=window, split_tokens=split)
        assert _close(out, ref) < 1e-12


def test_window_of_one_returns_own_value_row(oracle_lib):
    """w = 1: each position sees only itself, so O = v_p exactly."""
    shape = wl.AttnShape(Hq=4, Hkv=2, d=32, P=16, S=64)
    lens = [70, 33]
    seqs = wl.make_sequences(lens)
    layout = wl.layout_pages(3, lens, shape.P)
    out, *_ = osd.run_oracle(shape, seqs, layout, 0, lens, window=1)
    want = np.concatenate([s.v(0, shape).to(torch.float64).numpy().repeat(shape.g, axis=1) for s in seqs])
    assert np.array_equal(out, want)


def test_window_wider_than_context_equals_full_attention(oracle_lib):
    shape = wl.AttnShape(Hq=8, Hkv=2, d=64, P=16, S=128)
    lens = list(wl.TINY_LENS)
    seqs = wl.make_sequences(lens)
    layout = wl.layout_pages(3, lens, shape.P)
    full, *_ = osd.run_oracle(shape, seqs, layout, 0, lens)
    for w in (300, 301, 10_000):
        out, *_ = osd.run_oracle(shape, seqs, layout, 0, lens, window=w)
        assert np.array_equal(out, full)


def test_window_zero_query_gives_mean_of_window(oracle_lib):
    shape = wl.AttnShape(Hq=2, Hkv=1, d=16, P=4, S=64)
    rng = np.random.default_rng(5)
    n, w = 23, 6
    K = _bf16(rng.standard_normal((n, 1, 16)))
    V = _bf16(rng.standard_normal((n, 1, 16)))
    Q = _bf16(np.zeros((n, 2, 16)))
    kc, vc = osd.host_pools(shape, 6)
    pos = np.arange(n)
    oracle.kv_append(osd.bits16(K), osd.bits16(V), pos, kc, vc, Hkv=1, d=16, P=4)
    out = oracle.paged_attention(osd.bits16(Q), np.array([0, n], np.int32), np.array([n], np.int32), kc, vc,
                                 np.arange(6, dtype=np.int32)[None, :], Hq=2, Hkv=1, d=16, P=4,
                                 scale=shape.scale, window=w)
    Vd = V.to(torch.float64).numpy()[:, 0, :]
    for i in range(n):
        mean = Vd[max(0, i - w + 1):i + 1].mean(axis=0)
        assert np.max(np.abs(out[i, 0] - mean)) < 1e-14


def test_window_page_permutation_is_bit_identical(oracle_lib):
    shape = wl.AttnShape(Hq=8, Hkv=2, d=64, P=16, S=128)
    lens = list(wl.TINY_LENS)
    seqs = wl.make_sequences(lens)
    a, *_ = osd.run_oracle(shape, seqs, wl.layout_pages(3, lens, shape.P), 0, lens, window=77)
    b, *_ = osd.run_oracle(shape, seqs, wl.layout_pages(8, lens, shape.P), 0, lens, window=77)
    assert np.array_equal(a, b)
