"""The split-KV decode demonstration of "Deterministic inference: results independent of the
batch" (section "The root: the order of floating-point additions"), restated in numpy fp32:
a split count chosen from the load (max(1, min(64, sms // batch)), 132 SMs) changes one
request's bits as the batch grows, while splitting at a fixed 2048 tokens gives the same 4
splits -- and the same bits -- at every batch size, within float error of the unsplit result.
The printed outcomes of that page are the pins, kept in tests/golden/handbook_split_kv_demo.txt
(64/8/2/1 splits; batch 16/64/256 differ from batch 1; fixed splits all equal and
allclose(atol=1e-5) to unsplit)."""
import numpy as np

from tests import golden


def _decode(q, K, V, n_splits):
    D = q.shape[0]
    parts = []
    for Kc, Vc in zip(np.array_split(K, n_splits), np.array_split(V, n_splits)):
        s = (Kc @ q) / np.float32(np.sqrt(D))
        m = s.max()
        p = np.exp(s - m)
        parts.append((m, p.sum(dtype=np.float32), p @ Vc))
    M = max(m for m, _, _ in parts)
    num = sum(np.exp(m - M) * o for m, _, o in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    return num / den


def _splits_by_load(batch, sms=132):
    return max(1, min(64, sms // batch))


def _splits_fixed(seq_len, tile=2048):
    return -(-seq_len // tile)


def test_load_based_split_changes_bits_fixed_split_does_not():
    fix = golden.load("handbook_split_kv_demo.txt")
    D, S = int(golden.one(fix, "head_dim")), int(golden.one(fix, "keys"))
    sms, tile = int(golden.one(fix, "sms")), int(golden.one(fix, "fixed_split_tokens"))
    rng = np.random.default_rng(0)
    q = rng.standard_normal(D).astype(np.float32)
    K = rng.standard_normal((S, D)).astype(np.float32)
    V = rng.standard_normal((S, D)).astype(np.float32)
    ref = _decode(q, K, V, _splits_by_load(1, sms))
    for row in fix["load"]:
        batch = int(row["batch"])
        assert _splits_by_load(batch, sms) == int(row["splits"])
        same = np.array_equal(_decode(q, K, V, _splits_by_load(batch, sms)), ref)
        assert same == golden.flag(row["equal_to_batch1"]), batch
    (frow,) = fix["fixed"]
    assert _splits_fixed(S, tile) == int(frow["splits"])
    fixed = [_decode(q, K, V, _splits_fixed(S, tile)) for _ in golden.ints(frow["batches"])]
    assert all(np.array_equal(f, fixed[0]) for f in fixed) == golden.flag(frow["all_equal"])
    s = (K @ q) / np.float32(np.sqrt(D))
    w = np.exp(s - s.max())
    unsplit = (w / w.sum()) @ V
    atol = float(golden.one(fix, "allclose_atol"))
    assert np.allclose(fixed[0], unsplit, atol=atol) == golden.flag(frow["allclose_to_unsplit"])
