"""The library's C++ page table (through the C ABI) against the Python reference model: identical
integer results -- cached lengths, write slots, block tables, refcounts, published flags, free
counts, eviction counts and status codes -- on the Vosti Figure 2 scenario and on random
operation sequences, with the normal rolling hash and with every page forced into one hash
bucket (collisions must never justify reuse)."""
import random

import pytest

from invariant_attention_amd import binding as ia
from oracle import pagepool as model


class Pair:
    def __init__(self, num_pages, P, flags=0):
        self.lib = ia.Pool(num_pages, P, flags)
        self.ref = model.PagePool(num_pages, P)
        self.n = num_pages

    def check_pages(self):
        for pg in range(self.n):
            assert ia.ia_pool_page_refs(self.lib, pg) == self.ref.page_refs(pg), pg
            assert ia.ia_pool_page_published(self.lib, pg) == int(self.ref.is_published(pg)), pg
        assert ia.ia_pool_num_free(self.lib) == self.ref.num_free()


def _lib_status(fn, *args):
    try:
        return ia.IA_OK, fn(*args)
    except ia.IAError as e:
        return e.status, None


@pytest.mark.parametrize("flags", [0, ia.IA_POOL_CONSTANT_HASH], ids=["hash", "constant-hash"])
def test_figure2_scenario_matches_model(flags):
    pp = Pair(8, 2, flags)
    seqs = []
    for toks in ([1, 2, 3, 4], [1, 2, 5, 6]):
        s_lib, c_lib = ia.ia_seq_begin(pp.lib, toks)
        st, s_ref, c_ref = pp.ref.seq_begin(toks)
        assert c_lib == c_ref
        sl = ia.ia_seq_reserve(pp.lib, s_lib, len(toks) - c_lib)
        st, sr = pp.ref.seq_reserve(s_ref, len(toks) - c_ref)
        assert sl == sr
        ia.ia_seq_commit(pp.lib, s_lib, len(toks) - c_lib)
        pp.ref.seq_commit(s_ref, len(toks) - c_ref)
        assert ia.ia_seq_block_table(s_lib) == pp.ref.seq_block_table(s_ref)
        seqs.append((s_lib, s_ref))
        pp.check_pages()
    for s_lib, s_ref in seqs:
        ia.ia_seq_end(pp.lib, s_lib)
        pp.ref.seq_end(s_ref)
        pp.check_pages()
    assert ia.ia_pool_evict(pp.lib, 1) == pp.ref.evict(1) == 1
    pp.check_pages()
    s_lib, c_lib = ia.ia_seq_begin(pp.lib, [1, 2, 3, 4])
    st, s_ref, c_ref = pp.ref.seq_begin([1, 2, 3, 4])
    assert c_lib == c_ref == 2
    assert ia.ia_seq_reserve(pp.lib, s_lib, 2) == pp.ref.seq_reserve(s_ref, 2)[1]
    pp.check_pages()


@pytest.mark.parametrize("seed", range(30))
def test_random_operations_match_model(seed):
    rng = random.Random(seed)
    P = rng.choice([2, 4, 16])
    flags = ia.IA_POOL_CONSTANT_HASH if seed % 3 == 0 else 0
    pp = Pair(rng.randint(4, 40), P, flags)
    vocab = rng.choice([2, 3, 50])
    base = [[rng.randint(1, vocab) for _ in range(rng.randint(1, 5 * P))] for _ in range(5)]
    live = []
    for step in range(150):
        op = rng.random()
        if op < 0.25 and len(live) < 6:
            toks = rng.choice(base) + [rng.randint(1, vocab) for _ in range(rng.randint(0, P))]
            s_lib, c_lib = ia.ia_seq_begin(pp.lib, toks)
            st, s_ref, c_ref = pp.ref.seq_begin(toks)
            assert c_lib == c_ref
            live.append([s_lib, s_ref, len(toks)])
        elif op < 0.55 and live:
            i = rng.randrange(len(live))
            s_lib, s_ref, hist = live[i]
            if s_ref.reserved == hist:
                t = [rng.randint(1, vocab) for _ in range(rng.randint(1, 3))]
                ia.ia_seq_append_tokens(pp.lib, s_lib, t)
                pp.ref.seq_append_tokens(s_ref, t)
                hist += len(t)
                live[i][2] = hist
            n_new = rng.randint(1, hist - s_ref.reserved)
            st_l, sl = _lib_status(ia.ia_seq_reserve, pp.lib, s_lib, n_new)
            st_r, sr = pp.ref.seq_reserve(s_ref, n_new)
            assert st_l == st_r
            if st_l == ia.IA_OK:
                assert sl == sr
        elif op < 0.75 and live:
            s_lib, s_ref, _ = rng.choice(live)
            if s_ref.reserved > s_ref.computed:
                k = rng.randint(1, s_ref.reserved - s_ref.computed)
                ia.ia_seq_commit(pp.lib, s_lib, k)
                pp.ref.seq_commit(s_ref, k)
                assert ia.ia_seq_len(s_lib) == s_ref.computed
        elif op < 0.88 and live:
            s_lib, s_ref, _ = live.pop(rng.randrange(len(live)))
            assert ia.ia_seq_block_table(s_lib) == pp.ref.seq_block_table(s_ref)
            ia.ia_seq_end(pp.lib, s_lib)
            pp.ref.seq_end(s_ref)
        else:
            want = rng.randint(1, 4)
            assert ia.ia_pool_evict(pp.lib, want) == pp.ref.evict(want)
        for s_lib, s_ref, _ in live:
            assert ia.ia_seq_block_table(s_lib) == pp.ref.seq_block_table(s_ref)
        pp.check_pages()
    for s_lib, s_ref, _ in live:
        ia.ia_seq_end(pp.lib, s_lib)


def test_invalid_arguments():
    pool = ia.Pool(4, 2)
    with pytest.raises(ia.IAError) as e:
        ia.ia_seq_begin(pool, [])
    assert e.value.status == ia.IA_ERR_INVALID_ARG
    s, c = ia.ia_seq_begin(pool, [1, 2, 3])
    with pytest.raises(ia.IAError):
        ia.ia_seq_reserve(pool, s, 4)  # past the history
    with pytest.raises(ia.IAError):
        ia.ia_seq_commit(pool, s, 1)  # nothing reserved
    with pytest.raises(ia.IAError) as e:
        ia.Pool(0, 16)
    ia.ia_seq_end(pool, s)
