"""Pins of the page-allocator oracle (oracle/page_pool.py): a hand-worked
example, invariants under random operation sequences (reference counts,
states, index, and a shadow model of what every page holds), LRU eviction
order, the dedup workload's page count, defragmentation preserving what every
table reads, and mutants that each of these catches."""

import json
import os

import numpy as np
import pytest

from oracle import page_pool as pp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pool_worked.json")


def expand(spec):
    out = []
    for part in spec:
        if part[0] == "range":
            out += list(range(part[1], part[2]))
        else:
            out += [part[1]] * part[2]
    return out


def replay(pool_cls=pp.PagePool):
    g = json.load(open(GOLDEN))
    prompts = {k: expand(v) for k, v in g["prompts"].items()}
    pool = pool_cls(g["num_pages"])
    for st in g["steps"]:
        op = st["op"]
        if op == "admit":
            pages, cached = pool.admit(prompts[st["prompt"]])
            assert pages == st["pages"], (st, pages)
            assert cached == st["cached_tokens"], (st, cached)
        elif op == "admit_fails":
            with pytest.raises(ValueError):
                pool.admit(prompts[st["prompt"]])
        elif op == "release":
            pool.release(st["pages"])
        elif op == "defrag":
            remap, moves = pool.defrag(st["move_referenced"])
            assert [list(m) for m in moves] == st["moves"]
            assert remap == st["remap"]
        assert list(pool.stats()) == st["stats"], (st, pool.stats())
    return pool


def test_worked_example():
    replay()


def test_defrag_of_referenced_pages_example():
    g = json.load(open(GOLDEN))["defrag_referenced"]
    pool = pp.PagePool(g["num_pages"])
    assert [pool.alloc(2) for _ in range(2)] == g["alloc"]
    pool.release(g["release"])
    remap, moves = pool.defrag(move_referenced=True)
    assert [list(m) for m in moves] == g["moves"] and remap == g["remap"]
    assert pp.remap_table(np.array(g["table_before"]), remap).tolist() == g["table_after"]


def check_invariants(pool, held):
    """held: list of page lists, one per reference holder."""
    refs = [0] * pool.P
    for pages in held:
        for p in pages:
            refs[p] += 1
    assert refs == pool.ref
    for p in range(pool.P):
        st = pool.state[p]
        assert (st == pp.USED) == (pool.ref[p] > 0)
        if st == pp.CACHED:
            assert pool.key[p] is not None and pool.index[pool.key[p]] == p
        if st == pp.FREE:
            assert pool.key[p] is None
    for k, p in pool.index.items():
        assert pool.key[p] == k and pool.state[p] != pp.FREE
    assert sum(pool.stats()) == pool.P


PREFIXES = [list(range(100, 100 + 700)), list(range(5000, 5000 + 520)), [3] * 900]


def random_prompt(rng):
    base = PREFIXES[int(rng.integers(0, len(PREFIXES)))]
    cut = int(rng.integers(1, len(base) + 1))
    tail = rng.integers(0, 50, int(rng.integers(0, 300))).tolist()
    return base[:cut] + tail


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_keep_invariants_and_contents(seed):
    """Random admissions (prompts sharing prefixes), releases, private
    allocations and defragmentations. Besides the bookkeeping invariants, a
    shadow copy of what each page holds (the prefix it was filled with) must
    agree with every reuse: a job never gets a page holding another prefix."""
    rng = np.random.default_rng(seed)
    P = 24
    pool = pp.PagePool(P)
    content = [None] * P          # shadow: tokens a page holds
    jobs = []                     # (pages, tokens)
    privs = []                    # private page lists
    for step in range(400):
        r = rng.random()
        if r < 0.45:
            toks = random_prompt(rng)
            try:
                pages, cached = pool.admit(toks)
            except ValueError:
                assert -(-len(toks) // 256) > pool.allocatable()
                continue
            assert cached % 256 == 0 and cached < len(toks)
            for j, p in enumerate(pages):
                want = tuple(toks[j * 256:(j + 1) * 256])
                if j * 256 < cached:
                    assert content[p] == tuple(toks[:(j + 1) * 256]), "reused page holds another prefix"
                else:
                    content[p] = tuple(toks[:(j + 1) * 256]) if len(want) == 256 else ("private", step, j)
            jobs.append((pages, toks))
        elif r < 0.75 and jobs:
            pages, _ = jobs.pop(int(rng.integers(0, len(jobs))))
            pool.release(pages)
        elif r < 0.85:
            n = int(rng.integers(0, 4))
            if n <= pool.allocatable():
                ps = pool.alloc(n)
                for p in ps:
                    content[p] = ("private", step, p)
                privs.append(ps)
        elif r < 0.92 and privs:
            pool.release(privs.pop())
        else:
            ref_move = bool(rng.integers(0, 2))
            remap, moves = pool.defrag(ref_move)
            moved_used = False
            for src, dst in moves:
                assert pool.state[dst] != pp.FREE and pool.state[src] == pp.FREE
                content[dst] = content[src]
                moved_used |= pool.state[dst] == pp.USED
            assert ref_move or not moved_used
            jobs = [([remap[p] for p in pages], toks) for pages, toks in jobs]
            privs = [[remap[p] for p in ps] for ps in privs]
            if ref_move:
                occ = sum(1 for s in pool.state if s != pp.FREE)
                assert all(pool.state[p] != pp.FREE for p in range(occ))
        check_invariants(pool, [pg for pg, _ in jobs] + privs)


def test_cached_prompt_keeps_one_token_to_prefill():
    """A prompt cached in full is matched up to its last full page minus one:
    the prefill keeps a token and never writes into a shared page."""
    pool = pp.PagePool(8)
    toks = list(range(512))
    pages, cached = pool.admit(toks)
    assert cached == 0
    pool.release(pages)
    again, cached = pool.admit(toks)
    assert cached == 256 and again[0] == pages[0] and again[1] != pages[1]


def test_least_recently_released_cached_page_is_evicted_first():
    pool = pp.PagePool(4)
    a, _ = pool.admit(list(range(300)))          # pages 0 (keyed), 1
    b, _ = pool.admit(list(range(1000, 1300)))   # pages 2 (keyed), 3
    pool.release(b)                              # page 2 cached first (older)
    pool.release(a)                              # page 0 cached second
    c, _ = pool.admit(list(range(2000, 2300)))   # free pages 1, 3 first ...
    assert c == [1, 3]
    d, _ = pool.admit([9] * 10)                  # ... then the older cached page, 2
    assert d == [2]
    pool.release(c)
    _, cached = pool.admit(list(range(301)))     # page 0 is still cached
    assert cached == 256


def test_dedup_workload_shares_the_prefix_pages():
    """100 jobs with one 4096-token prefix and private tails of 1..256 tokens
    (the shape of the dedup configuration) fit a 256-page pool as 16 shared
    pages plus one private page each; every job after the first finds the
    prefix cached."""
    rng = np.random.default_rng(4)
    pool = pp.PagePool(256)
    prefix = rng.integers(0, 128000, 4096).tolist()
    for i in range(100):
        tail = rng.integers(0, 128000, int(rng.integers(1, 257))).tolist()
        pages, cached = pool.admit(prefix + tail)
        assert len(pages) == 17 and cached == (0 if i == 0 else 4096)
    assert pool.stats() == (256 - 116, 0, 116)
    assert max(pool.ref) == 100


def test_defrag_keeps_what_every_table_reads():
    rng = np.random.default_rng(8)
    P, Hkv, D = 20, 2, 4
    pool = pp.PagePool(P)
    jobs = []
    for _ in range(30):
        try:
            jobs.append(pool.admit(random_prompt(rng))[0])
        except ValueError:
            break
        if len(jobs) > 2 and rng.random() < 0.5:
            pool.release(jobs.pop(0))
    k = rng.integers(0, 2**16, (P, Hkv, 256, D), dtype=np.uint16)
    v = rng.integers(0, 2**16, (P, Hkv, 256, D), dtype=np.uint16)
    W = max(len(j) for j in jobs)
    table = np.full((len(jobs), W), -1, np.int32)
    for b, pages in enumerate(jobs):
        table[b, :len(pages)] = pages
    before = [k[table[b][table[b] >= 0]] for b in range(len(jobs))]
    remap, moves = pool.defrag(move_referenced=True)
    k2, v2 = pp.copy_pages(k, v, moves)
    t2 = pp.remap_table(table, remap)
    for b in range(len(jobs)):
        assert np.array_equal(k2[t2[b][t2[b] >= 0]], before[b])
    occ = sum(1 for s in pool.state if s != pp.FREE)
    assert sorted(set(t2[t2 >= 0].tolist())) == sorted(set(t2[t2 >= 0].tolist()) & set(range(occ)))


# ------------------------------------------------------------------ mutants

Base = pp.PagePool   # the oracle's class, kept while the battery swaps it out


class EvictNewest(Base):
    def _take(self):
        for p in range(self.P):
            if self.state[p] == pp.FREE:
                return p
        best = max((p for p in range(self.P) if self.state[p] == pp.CACHED), key=lambda p: self.stamp[p])
        del self.index[self.key[best]]
        self.key[best] = None
        self.state[best] = pp.FREE
        return best


class CachedBeforeFree(Base):
    def _take(self):
        cached = [p for p in range(self.P) if self.state[p] == pp.CACHED]
        if cached:
            best = min(cached, key=lambda p: self.stamp[p])
            del self.index[self.key[best]]
            self.key[best] = None
            self.state[best] = pp.FREE
            return best
        return Base._take(self)


class NoPromptCache(Base):
    def release(self, pages):
        Base.release(self, pages)
        for p in range(self.P):
            if self.state[p] == pp.CACHED:
                del self.index[self.key[p]]
                self.key[p] = None
                self.state[p] = pp.FREE


class MatchWholePrompt(Base):
    def admit(self, tokens):
        # matches the last full page too (no token left to prefill)
        tokens = list(tokens)
        n = len(tokens)
        extra = [0] if n % 256 == 0 and n > 0 else []
        pages, cached = Base.admit(self, tokens + extra)
        if extra and len(pages) > -(-n // 256):
            self.release([pages[-1]])
            pages = pages[:-1]
        return pages, cached


class DefragWithoutReindex(Base):
    def defrag(self, move_referenced=False):
        index = dict(self.index)
        remap, moves = Base.defrag(self, move_referenced)
        self.index = index
        return remap, moves


class NotAllOrNothing(Base):
    def admit(self, tokens):
        try:
            return Base.admit(self, tokens)
        except ValueError:
            self.alloc(min(self.allocatable(), 1))
            raise


MUTANTS = [EvictNewest, CachedBeforeFree, NoPromptCache, MatchWholePrompt, DefragWithoutReindex, NotAllOrNothing]


def battery(cls):
    """Every pin above, on a pool class."""
    def run(f):
        try:
            f()
            return True
        except (AssertionError, ValueError, KeyError, TypeError):
            return False
    orig = pp.PagePool
    pp.PagePool = cls
    try:
        ok = [run(lambda: replay(cls)), run(test_cached_prompt_keeps_one_token_to_prefill),
              run(test_least_recently_released_cached_page_is_evicted_first),
              run(test_dedup_workload_shares_the_prefix_pages)]
        ok += [run(lambda s=s: test_random_operations_keep_invariants_and_contents(s)) for s in range(3)]
    finally:
        pp.PagePool = orig
    return all(ok)


def test_the_battery_passes_on_the_oracle():
    assert battery(pp.PagePool)


@pytest.mark.parametrize("cls", MUTANTS, ids=[c.__name__ for c in MUTANTS])
def test_each_mutant_fails_the_battery(cls):
    assert not battery(cls)
