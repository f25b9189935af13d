"""The opt-in host validators of the C ABI (no GPU): ia_validate_slots (write isolation, Vosti
§4.3) and ia_validate_attention_args (lengths and block-table entries, Vosti App. A.1)."""
import numpy as np
import pytest

from invariant_attention_amd import binding as ia


def _status(fn, *args, **kw):
    try:
        fn(*args, **kw)
        return ia.IA_OK
    except ia.IAError as e:
        return e.status


def test_slots_without_pool():
    assert _status(ia.ia_validate_slots, None, [0, 1, 17, -1, -5], 4, 16) == ia.IA_OK
    assert _status(ia.ia_validate_slots, None, [], 4, 16) == ia.IA_OK
    assert _status(ia.ia_validate_slots, None, [3, 64], 4, 16) == ia.IA_ERR_INVALID_ARG  # past the pool
    assert _status(ia.ia_validate_slots, None, [3, 7, 3], 4, 16) == ia.IA_ERR_INVALID_ARG  # written twice
    assert _status(ia.ia_validate_slots, None, [-1, -1], 4, 16) == ia.IA_OK  # padding rows may repeat


def test_slots_on_published_page_are_refused():
    pool = ia.Pool(6, 2)
    s, cached = ia.ia_seq_begin(pool, [5, 6, 7, 8, 9])
    slots = ia.ia_seq_reserve(pool, s, 5)
    ia.ia_validate_slots(pool, slots, 6, 2)  # the pool's own slots pass
    ia.ia_seq_commit(pool, s, 5)  # pages of [5, 6] and [7, 8] are published
    assert _status(ia.ia_validate_slots, pool, [slots[0]], 6, 2) == ia.IA_ERR_PAGE_REFERENCED
    assert _status(ia.ia_validate_slots, pool, [slots[3]], 6, 2) == ia.IA_ERR_PAGE_REFERENCED
    assert _status(ia.ia_validate_slots, pool, [slots[4]], 6, 2) == ia.IA_OK  # the partial page stays private
    assert _status(ia.ia_validate_slots, pool, [slots[4]], 7, 2) == ia.IA_ERR_INVALID_ARG  # wrong pool size
    ia.ia_seq_end(pool, s)


def test_attention_args():
    bt = np.array([[3, 1, 0, -1], [2, 4, -1, -1]], np.int32)
    seq_lens = np.array([40, 20], np.int32)
    ok = dict(num_pages=5, page_size=16, max_seq_len=64)
    ia.ia_validate_attention_args(None, seq_lens, bt, **ok)  # decode
    ia.ia_validate_attention_args(np.array([0, 3, 23], np.int32), seq_lens, bt, **ok)  # prefill chunk + whole
    bad = [
        ((np.array([0, 3, 24], np.int32), seq_lens, bt), ok),           # q_len 21 > seq_len 20
        ((np.array([1, 3, 23], np.int32), seq_lens, bt), ok),           # cu_q_lens[0] != 0
        ((np.array([0, 0, 20], np.int32), seq_lens, bt), ok),           # an empty query
        ((None, np.array([40, 70], np.int32), bt), ok),                 # past max_seq_len
        ((None, np.array([40, 33], np.int32), bt), ok),                 # 3 pages, entry -1
        ((None, seq_lens, np.array([[3, 1, 5], [2, 4, 0]], np.int32)), ok),  # page 5 of 5
        ((None, np.array([65, 1], np.int32), bt), dict(ok, max_seq_len=80)),  # 5 pages > 4 entries
    ]
    for args, kw in bad:
        assert _status(ia.ia_validate_attention_args, *args, **kw) == ia.IA_ERR_INVALID_ARG, (args, kw)
