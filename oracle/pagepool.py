"""Reference model of the paged, prefix-sharing KV page pool -- TEST INFRASTRUCTURE ONLY.

A plain Python model of the host page layer, used as the oracle for the
library's C++ page table (integer results must agree exactly).  It follows
Vosti: Specifying, Implementing, and Verifying Deterministic LLM Inference,
§4.1-§4.3 and Figure 2:

* A cached page is reused only for the token prefix that produced it: the
  candidate must hold the same tokens, sit at the same depth of the prefix
  and hang off the same physical parent page ("Exact prefix matching").  The
  model finds candidates by exhaustive search, so no hash can stand in for
  the exact check.
* Cache hits are resolved when a sequence begins, before it registers any
  page it will produce; new values go to private suffix pages; a page is
  published for reuse only once it is full and computed ("Separate cache
  reuse from generation", "State updates").
* Shared and published pages are immutable; write slots are private and
  disjoint ("Sharing and write isolation").
* Under memory pressure only unreferenced leaves of the parent chain are
  evicted, so a parent is never recycled while a retained child refers to it.

Readings taken where the pages leave a choice open (the C++ layer makes the
same ones): free pages are handed out lowest id first; eviction takes the
least recently released unreferenced leaf (ties by page id); at least one
prompt token is always left to compute, so a fully cached prompt re-computes
its last page; a page whose parent page is not published is not published
itself, and a full page identical to one already published stays private.
"""
from __future__ import annotations

OK = 0
ERR_INVALID_ARG = 1
ERR_OUT_OF_PAGES = 4


class _Seq:
    def __init__(self, tokens):
        self.history = list(tokens)
        self.pages: list[int] = []
        self.reserved = 0
        self.computed = 0
        self.live = True


class PagePool:
    def __init__(self, num_pages: int, page_size: int):
        if num_pages <= 0 or page_size <= 0:
            raise ValueError("bad pool size")
        self.P = page_size
        self.num_pages = num_pages
        self.free = set(range(num_pages))
        self.refs = [0] * num_pages
        # published page -> (parent page or -1, depth, tokens)
        self.published: dict[int, tuple[int, int, tuple]] = {}
        self.released_at: dict[int, int] = {}
        self.clock = 0

    # ----------------------------------------------------------- helpers
    def _find(self, parent: int, depth: int, tokens: tuple) -> int | None:
        for page, rec in self.published.items():
            if rec == (parent, depth, tokens):
                return page
        return None

    def _has_published_child(self, page: int) -> bool:
        return any(rec[0] == page for rec in self.published.values())

    def _alloc(self) -> int:
        page = min(self.free)
        self.free.remove(page)
        return page

    # -------------------------------------------------------------- API
    def seq_begin(self, tokens):
        """Attach the longest exactly matching published prefix; returns (seq, cached_len)."""
        tokens = list(tokens)
        if len(tokens) == 0:
            return ERR_INVALID_ARG, None, 0
        seq = _Seq(tokens)
        parent = -1
        P = self.P
        depth = 0
        while (depth + 1) * P < len(tokens):
            blk = tuple(tokens[depth * P:(depth + 1) * P])
            page = self._find(parent, depth, blk)
            if page is None:
                break
            self.refs[page] += 1
            self.released_at.pop(page, None)
            seq.pages.append(page)
            parent = page
            depth += 1
        seq.reserved = seq.computed = depth * P
        return OK, seq, seq.computed

    def seq_append_tokens(self, seq, tokens):
        if not seq.live:
            return ERR_INVALID_ARG
        seq.history.extend(tokens)
        return OK

    def seq_reserve(self, seq, n_new: int):
        """Slots (page * P + offset) for the next n_new history positions."""
        if not seq.live or n_new < 0 or seq.reserved + n_new > len(seq.history):
            return ERR_INVALID_ARG, []
        P = self.P
        need = -(-(seq.reserved + n_new) // P) - len(seq.pages)
        if need > len(self.free):
            self.evict(need - len(self.free))
        if need > len(self.free):
            return ERR_OUT_OF_PAGES, []
        for _ in range(max(need, 0)):
            page = self._alloc()
            self.refs[page] = 1
            seq.pages.append(page)
        slots = [seq.pages[pos // P] * P + pos % P for pos in range(seq.reserved, seq.reserved + n_new)]
        seq.reserved += n_new
        return OK, slots

    def seq_commit(self, seq, n_done: int):
        """Mark n_done reserved positions computed and publish pages that became full."""
        if not seq.live or n_done < 0 or seq.computed + n_done > seq.reserved:
            return ERR_INVALID_ARG
        seq.computed += n_done
        P = self.P
        for i in range(seq.computed // P):
            page = seq.pages[i]
            if page in self.published:
                continue
            parent = seq.pages[i - 1] if i > 0 else -1
            if parent != -1 and parent not in self.published:
                break
            blk = tuple(seq.history[i * P:(i + 1) * P])
            if self._find(parent, i, blk) is not None:
                break  # identical page already published: keep this copy private
            self.published[page] = (parent, i, blk)
        return OK

    def seq_block_table(self, seq):
        return list(seq.pages)

    def seq_end(self, seq):
        if not seq.live:
            return ERR_INVALID_ARG
        for page in seq.pages:
            self.refs[page] -= 1
            if page in self.published:
                if self.refs[page] == 0:
                    self.released_at[page] = self.clock
                    self.clock += 1
            else:
                self.refs[page] = 0
                self.free.add(page)
        seq.pages = []
        seq.live = False
        return OK

    def evict(self, want: int) -> int:
        """Evict up to `want` unreferenced published leaves, least recently released first."""
        done = 0
        while done < want:
            cands = [p for p in self.published
                     if self.refs[p] == 0 and not self._has_published_child(p)]
            if not cands:
                break
            victim = min(cands, key=lambda p: (self.released_at[p], p))
            del self.published[victim]
            del self.released_at[victim]
            self.free.add(victim)
            done += 1
        return done

    # ------------------------------------------------------ introspection
    def page_refs(self, page: int) -> int:
        return self.refs[page]

    def is_published(self, page: int) -> bool:
        return page in self.published

    def num_free(self) -> int:
        return len(self.free)
