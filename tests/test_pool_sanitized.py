"""The host page table under AddressSanitizer and UndefinedBehaviorSanitizer.

csrc/pool.cpp is compiled on its own (host code only, g++) together with tests/pool_replay.cpp, a
driver that reads operations from stdin, and replayed over the Vosti Figure 2 scenario and over
random operation sequences (the same generator as the ABI test).  Every result line must equal
what the page-pool model gives, and the sanitizers must report nothing (the build aborts on the
first report).  The opt-in slot validator (Vosti §4.3, write isolation) is exercised in the same
replays: slots the pool hands out always pass it, a slot on a published page is refused with
IA_ERR_PAGE_REFERENCED, and repeated or out-of-range slots with IA_ERR_INVALID_ARG."""
from __future__ import annotations

import os
import random
import shutil
import subprocess

import pytest

from oracle import pagepool as model

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, PAGE_REFERENCED = 0, 1, 5


@pytest.fixture(scope="module")
def replay_bin(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    out = str(tmp_path_factory.mktemp("pool_asan") / "pool_replay")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", os.path.join(ROOT, "tests", "pool_replay.cpp"),
           os.path.join(ROOT, "invariant_attention_amd", "csrc", "pool.cpp"), "-o", out]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0 and "asan" in proc.stderr.lower():
        pytest.skip("the sanitizer runtime is not installed: " + proc.stderr[-300:])
    assert proc.returncode == 0, proc.stderr
    return out


def _run(binary, lines):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    proc = subprocess.run([binary], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env,
                          timeout=120)
    assert proc.returncode == 0, proc.stderr[-4000:]
    assert "runtime error" not in proc.stderr and "AddressSanitizer" not in proc.stderr, proc.stderr[-4000:]
    return proc.stdout.splitlines()


class Script:
    """Operations for the driver, with the model's expected result line for each."""

    def __init__(self, num_pages, P, flags=0):
        self.ref = model.PagePool(num_pages, P)
        self.n, self.P = num_pages, P
        self.ops = [f"create {num_pages} {P} {flags}"]
        self.want = ["create 0"]
        self.seqs = {}

    def _op(self, text, want):
        self.ops.append(text)
        self.want.append(want)

    def pages(self):
        cells = " ".join(f"{self.ref.page_refs(p)}:{int(self.ref.is_published(p))}" for p in range(self.n))
        self._op("pages", f"pages {self.ref.num_free()} {cells}")

    def begin(self, sid, toks):
        st, s, cached = self.ref.seq_begin(toks)
        self.seqs[sid] = s
        self._op(f"begin {sid} {len(toks)} " + " ".join(map(str, toks)), f"begin {st} {cached}")
        return s

    def append(self, sid, toks):
        st = self.ref.seq_append_tokens(self.seqs[sid], toks)
        self._op(f"append {sid} {len(toks)} " + " ".join(map(str, toks)), f"append {st}")

    def reserve(self, sid, n):
        st, slots = self.ref.seq_reserve(self.seqs[sid], n)
        self._op(f"reserve {sid} {n}", " ".join(["reserve", str(st)] + [str(x) for x in slots]))
        if st == OK and slots:
            # The pool's own slots always pass the validator.
            self.vslots(slots)
        return st, slots

    def commit(self, sid, n):
        st = self.ref.seq_commit(self.seqs[sid], n)
        self._op(f"commit {sid} {n}", f"commit {st}")

    def bt(self, sid):
        pages = self.ref.seq_block_table(self.seqs[sid])
        self._op(f"bt {sid}", " ".join(["bt", "0"] + [str(p) for p in pages]))
        self._op(f"len {sid}", f"len {self.seqs[sid].computed}")

    def end(self, sid):
        st = self.ref.seq_end(self.seqs.pop(sid))
        self._op(f"end {sid}", f"end {st}")

    def evict(self, want):
        self._op(f"evict {want}", f"evict 0 {self.ref.evict(want)}")

    def vslots(self, slots):
        # In slot order, the first slot past the pool or on a published page decides; failing
        # that, a slot that appears twice.
        limit = self.n * self.P
        st = OK
        for s in slots:
            if s < 0:
                continue
            if s >= limit:
                st = INVALID
                break
            if self.ref.is_published(s // self.P):
                st = PAGE_REFERENCED
                break
        used = [s for s in slots if s >= 0]
        if st == OK and len(set(used)) != len(used):
            st = INVALID
        self._op(f"vslots {len(slots)} " + " ".join(map(str, slots)), f"vslots {st}")


def test_figure2_under_sanitizers(replay_bin):
    sc = Script(8, 2)
    for sid, toks in enumerate(([1, 2, 3, 4], [1, 2, 5, 6])):
        s = sc.begin(sid, toks)
        sc.reserve(sid, len(toks) - s.computed)
        sc.commit(sid, len(toks) - s.computed)
        sc.bt(sid)
        sc.pages()
    # A and B share the published first page: writing it again is refused.
    shared = sc.ref.seq_block_table(sc.seqs[0])[0]
    sc.vslots([shared * 2 + 1])
    sc.vslots([-1, 3, 3])
    sc.vslots([8 * 2])
    for sid in (0, 1):
        sc.end(sid)
        sc.pages()
    sc.evict(1)
    sc.pages()
    s = sc.begin(2, [1, 2, 3, 4])
    assert s.computed == 2
    sc.reserve(2, 2)
    sc.pages()
    sc.end(2)
    assert _run(replay_bin, sc.ops) == sc.want


@pytest.mark.parametrize("seed", range(30))
def test_random_operations_under_sanitizers(replay_bin, seed):
    rng = random.Random(1000 + seed)
    P = rng.choice([2, 4, 16])
    sc = Script(rng.randint(4, 40), P, 1 if seed % 3 == 0 else 0)
    vocab = rng.choice([2, 3, 50])
    base = [[rng.randint(1, vocab) for _ in range(rng.randint(1, 5 * P))] for _ in range(5)]
    live = {}
    next_id = 0
    for _ in range(150):
        op = rng.random()
        if op < 0.25 and len(live) < 6:
            toks = rng.choice(base) + [rng.randint(1, vocab) for _ in range(rng.randint(0, P))]
            sc.begin(next_id, toks)
            live[next_id] = len(toks)
            next_id += 1
        elif op < 0.55 and live:
            sid = rng.choice(sorted(live))
            s = sc.seqs[sid]
            if s.reserved == live[sid]:
                t = [rng.randint(1, vocab) for _ in range(rng.randint(1, 3))]
                sc.append(sid, t)
                live[sid] += len(t)
            sc.reserve(sid, rng.randint(1, live[sid] - s.reserved))
        elif op < 0.75 and live:
            sid = rng.choice(sorted(live))
            s = sc.seqs[sid]
            if s.reserved > s.computed:
                sc.commit(sid, rng.randint(1, s.reserved - s.computed))
        elif op < 0.88 and live:
            sid = rng.choice(sorted(live))
            sc.bt(sid)
            sc.end(sid)
            del live[sid]
        else:
            sc.evict(rng.randint(1, 4))
        if rng.random() < 0.2:
            sc.vslots([rng.randint(-1, sc.n * P) for _ in range(rng.randint(1, 6))])
        sc.pages()
    for sid in sorted(live):
        sc.end(sid)
    assert _run(replay_bin, sc.ops) == sc.want
