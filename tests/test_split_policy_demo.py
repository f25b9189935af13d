"""Pin from the split-KV decode example of "Deterministic inference: results independent of the
batch" (section "The root: the order of floating-point additions").  The page runs one request
(head dim 64, 8192 keys) at several batch sizes and prints, for a split count picked from the load
and for a fixed 2048-token split, how many pieces the request's keys are cut into and whether the
result keeps its bits.  Those printed outcomes are in tests/golden/handbook_split_kv_demo.txt.

Here the same experiment runs on the oracle's own split mode, the fixed-length split with the
ascending merge that the GPU path implements: the request is decoded with the piece length each
policy gives at each batch size (8192 / k keys, k = the load-picked piece count; 2048 keys for the
fixed policy), and the printed outcomes are checked: the load-picked counts are 64 / 8 / 2 / 1, the
results at batch 16 / 64 / 256 differ from batch 1's, and the fixed split gives 4 pieces at every
batch size, the same bits each time, within the page's tolerance of the unsplit result."""
import numpy as np

from synth import workloads as wl
from tests import golden
from tests import oracle_side as osd


def _load_picked_pieces(batch: int, sms: int) -> int:
    # One piece per idle streaming multiprocessor, at least 1 and at most 64 (the page's heuristic).
    return max(1, min(64, sms // batch))


def _decode(shape, seqs, layout, split_tokens):
    out, _, _, _, _ = osd.run_oracle(shape, seqs, layout, 0, [1], split_tokens=split_tokens)
    return out


def test_load_picked_split_changes_bits_fixed_split_does_not():
    fix = golden.load("handbook_split_kv_demo.txt")
    d, n = int(golden.one(fix, "head_dim")), int(golden.one(fix, "keys"))
    sms, fixed_len = int(golden.one(fix, "sms")), int(golden.one(fix, "fixed_split_tokens"))
    shape = wl.AttnShape(Hq=1, Hkv=1, d=d, P=16, S=fixed_len)
    seqs = wl.make_sequences([n], first_sid=77)
    layout = wl.layout_pages(1, [n], shape.P)

    by_batch = {}
    for row in fix["load"]:
        batch = int(row["batch"])
        k = _load_picked_pieces(batch, sms)
        assert k == int(row["splits"]), batch
        assert n % k == 0
        by_batch[batch] = _decode(shape, seqs, layout, n // k)
    ref = by_batch[1]
    for row in fix["load"]:
        same = np.array_equal(by_batch[int(row["batch"])], ref)
        assert same == golden.flag(row["equal_to_batch1"]), row

    (frow,) = fix["fixed"]
    assert -(-n // fixed_len) == int(frow["splits"])
    fixed = [_decode(shape, seqs, layout, fixed_len) for _ in golden.ints(frow["batches"])]
    assert all(np.array_equal(f, fixed[0]) for f in fixed) == golden.flag(frow["all_equal"])
    unsplit = _decode(shape, seqs, layout, 0)
    atol = float(golden.one(fix, "allclose_atol"))
    assert np.allclose(fixed[0], unsplit, atol=atol, rtol=0) == golden.flag(frow["allclose_to_unsplit"])
