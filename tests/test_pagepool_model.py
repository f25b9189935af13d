"""Pins for the page-pool reference model: the sharing / retention / eviction / reuse scenario of
Vosti Figure 2 (two tokens a page), and the invariants of Vosti §4.2-4.3 checked after every step
of random operation sequences."""
import random

import pytest

from oracle.pagepool import ERR_OUT_OF_PAGES, OK, PagePool
from tests import golden

a, b, c, d, e, f = 1, 2, 3, 4, 5, 6


def _run(pool, tokens):
    st, seq, cached = pool.seq_begin(tokens)
    assert st == OK
    st, slots = pool.seq_reserve(seq, len(tokens) - cached)
    assert st == OK
    assert pool.seq_commit(seq, len(tokens) - cached) == OK
    return seq, cached, slots


def _refs(text):
    return {k: int(v) for k, v in (kv.split(":") for kv in text.split(","))}


def test_vosti_figure2_share_retain_evict_reuse():
    # Stage by stage against the reference counts Vosti Figure 2 prints
    # (tests/golden/vosti_figure2_page_states.txt).  The pool hands out its own page ids, so the
    # figure's pages are matched by role: the shared [a, b] page and the two suffix pages.
    fix = golden.load("vosti_figure2_page_states.txt")
    P = int(golden.one(fix, "page_size"))
    tok = {ch: i + 1 for i, ch in enumerate("abcdef")}
    req = {k: [tok[t] for t in v.split(",")] for r in fix["request"] for k, v in r.items()}
    stages = {int(st[""]): st for st in fix["stage"]}
    pool = PagePool(num_pages=8, page_size=P)
    A, cached_a, _ = _run(pool, req["A"])
    assert cached_a == 0
    B, cached_b, slots_b = _run(pool, req["B"])
    shared, a_suffix = pool.seq_block_table(A)
    shared_b, b_suffix = pool.seq_block_table(B)
    role = {"shared": shared, "A_suffix": a_suffix, "B_suffix": b_suffix}
    fig = {}
    for pg in fix["page"]:
        name = next(k for k in pg if k != "role")
        fig[name] = role[pg["role"]]

    def check(stage):
        for name, refs in _refs(stages[stage]["refs"]).items():
            assert pool.page_refs(fig[name]) == refs, (stage, name)
            assert pool.is_published(fig[name]), (stage, name)
        if "free" in stages[stage]:
            assert not pool.is_published(fig[stages[stage]["free"]]), stage

    # 1: A and B live, sharing the [a, b] page with private suffix pages
    assert cached_b == P and shared_b == shared
    check(1)
    assert all(s // P == b_suffix for s in slots_b)  # B writes only its private page
    # 2: both finish; pages are retained with refs 0
    pool.seq_end(A)
    pool.seq_end(B)
    check(2)
    # 3: evict one page -- a leaf goes (A's suffix, released first); the shared parent stays
    assert pool.evict(1) == 1
    check(3)
    leaves = [p for p in pool.published if pool.page_refs(p) == 0 and not pool._has_published_child(p)]
    assert shared not in leaves  # cannot go while B's suffix refers to it
    # 4: C reuses the shared page and recomputes its suffix into fresh storage
    st, C, cached_c = pool.seq_begin(req["C"])
    assert st == OK and cached_c == int(stages[4]["cached"])
    assert pool.seq_block_table(C) == [shared]
    check(4)
    n_new = len(stages[4]["recomputed"].split(","))
    st, slots = pool.seq_reserve(C, n_new)
    assert st == OK and len(slots) == n_new and len({s // P for s in slots}) == 1
    assert not pool.is_published(slots[0] // P)


def test_fully_cached_prompt_recomputes_last_page():
    pool = PagePool(num_pages=8, page_size=2)
    A, _, _ = _run(pool, [a, b, c, d])
    st, B, cached = pool.seq_begin([a, b, c, d])
    assert cached == 2  # at least one token is left to compute
    st, slots = pool.seq_reserve(B, 2)
    assert pool.seq_commit(B, 2) == OK
    # the recomputed page duplicates a published one and stays private
    assert not pool.is_published(slots[0] // 2)
    pool.seq_end(B)
    assert slots[0] // 2 in pool.free


def test_reuse_needs_same_parent_and_depth():
    pool = PagePool(num_pages=16, page_size=2)
    _run(pool, [a, b, c, d])
    # same tokens [c, d] at depth 1 but after a different parent: no reuse past the first page
    st, X, cached = pool.seq_begin([e, f, c, d, a])
    assert cached == 0
    # same tokens at a different depth: no reuse
    st, Y, cached = pool.seq_begin([c, d, a, b, a])
    assert cached == 0
    st, Z, cached = pool.seq_begin([a, b, c, d, e])
    assert cached == 4


def test_out_of_pages_is_an_error_without_allocation():
    pool = PagePool(num_pages=2, page_size=2)
    st, A, _ = pool.seq_begin([a, b, c, d, e])
    st, slots = pool.seq_reserve(A, 5)
    assert st == ERR_OUT_OF_PAGES and slots == [] and pool.num_free() == 2
    st, slots = pool.seq_reserve(A, 4)
    assert st == OK and pool.num_free() == 0


def _check_invariants(pool, live):
    # refcount = number of live sequences holding the page
    for pg in range(pool.num_pages):
        holders = sum(pg in s.pages for s in live)
        assert pool.refs[pg] == holders, pg
        if pg in pool.free:
            assert holders == 0 and pg not in pool.published
    # published records agree with every live history that holds them (canonical prefix)
    for s in live:
        for i, pg in enumerate(s.pages):
            if pg in pool.published:
                parent, depth, toks = pool.published[pg]
                assert depth == i and toks == tuple(s.history[i * pool.P:(i + 1) * pool.P])
                assert parent == (s.pages[i - 1] if i else -1)
    # parents of published pages are published (no dangling chain)
    for pg, (parent, depth, _) in pool.published.items():
        assert parent == -1 or parent in pool.published
    # private pages belong to exactly one live sequence
    for pg in range(pool.num_pages):
        if pg not in pool.free and pg not in pool.published:
            assert sum(pg in s.pages for s in live) == 1


@pytest.mark.parametrize("seed", range(12))
def test_random_operation_invariants(seed):
    rng = random.Random(seed)
    P = rng.choice([2, 4])
    pool = PagePool(num_pages=rng.randint(6, 24), page_size=P)
    prompts = [[rng.randint(1, 3) for _ in range(rng.randint(1, 14))] for _ in range(6)]
    live = []
    for _ in range(120):
        op = rng.random()
        if op < 0.3 and len(live) < 5:
            st, s, cached = pool.seq_begin(rng.choice(prompts) + [rng.randint(1, 3)] * rng.randint(0, 3))
            assert cached % P == 0 and cached < len(s.history)
            live.append(s)
        elif op < 0.6 and live:
            s = rng.choice(live)
            if s.reserved == len(s.history):
                pool.seq_append_tokens(s, [rng.randint(1, 3)])
            n_new = rng.randint(1, len(s.history) - s.reserved)
            before_free = set(pool.free)
            st, slots = pool.seq_reserve(s, n_new)
            if st == OK:
                pages = {x // P for x in slots}
                assert not (pages & set(pool.published))  # writes never hit published pages
                for o in live:
                    if o is not s:
                        assert not (pages & set(o.pages))  # nor another sequence's pages
            else:
                assert st == ERR_OUT_OF_PAGES
                assert before_free <= set(pool.free)
        elif op < 0.8 and live:
            s = rng.choice(live)
            if s.reserved > s.computed:
                assert pool.seq_commit(s, rng.randint(1, s.reserved - s.computed)) == OK
        elif op < 0.9 and live:
            s = live.pop(rng.randrange(len(live)))
            pool.seq_end(s)
        else:
            before = dict(pool.published)
            n = pool.evict(rng.randint(1, 3))
            gone = set(before) - set(pool.published)
            assert len(gone) == n
            for pg in gone:
                assert pool.refs[pg] == 0
                assert all(rec[0] != pg for rec in pool.published.values())
        _check_invariants(pool, live)
