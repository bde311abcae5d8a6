"""The library's page allocator (host code, no GPU) against the oracle: the
hand-worked example, random operation sequences with every decision compared
exactly (pages handed out, cached-token counts, failures, counts per state,
defragmentation plans), and the error paths."""

import json
import os

import numpy as np
import pytest

from oracle import page_pool as opool
from tests.test_oracle_pool import GOLDEN, expand, random_prompt


@pytest.fixture(scope="module")
def pk():
    import paged_kv_attention_attn_amd as pk
    return pk


class Lib:
    """The library pool with the oracle's method names."""

    def __init__(self, pk, P):
        self.pk, self.P = pk, P
        self.h = pk.pkv_pool_create(P)

    def __del__(self):
        self.pk.pkv_pool_destroy(self.h)

    def stats(self):
        return self.pk.pkv_pool_stats(self.h)

    def admit(self, toks):
        try:
            return self.pk.pkv_pool_admit(self.h, toks)
        except self.pk.PkvError as e:
            raise ValueError(str(e))

    def alloc(self, n):
        return self.pk.pkv_pool_alloc(self.h, n)

    def release(self, pages):
        self.pk.pkv_pool_release(self.h, pages)

    def retain(self, pages):
        self.pk.pkv_pool_retain(self.h, pages)

    def defrag(self, move_referenced=False):
        remap, moves = self.pk.pkv_pool_defrag(self.h, self.P, move_referenced)
        return remap, [tuple(m) for m in moves]


def test_worked_example(pk):
    g = json.load(open(GOLDEN))
    prompts = {k: expand(v) for k, v in g["prompts"].items()}
    pool = Lib(pk, g["num_pages"])
    for st in g["steps"]:
        if st["op"] == "admit":
            assert pool.admit(prompts[st["prompt"]]) == (st["pages"], st["cached_tokens"]), st
        elif st["op"] == "admit_fails":
            with pytest.raises(ValueError):
                pool.admit(prompts[st["prompt"]])
        elif st["op"] == "release":
            pool.release(st["pages"])
        elif st["op"] == "defrag":
            remap, moves = pool.defrag(st["move_referenced"])
            assert remap == st["remap"] and [list(m) for m in moves] == st["moves"]
        assert list(pool.stats()) == st["stats"], st


@pytest.mark.parametrize("seed", range(8))
def test_random_operations_match_the_oracle(pk, seed):
    rng = np.random.default_rng(100 + seed)
    P = 24 if seed % 2 else 40
    ref, lib = opool.PagePool(P), Lib(pk, P)
    jobs, privs = [], []
    for step in range(500):
        r = rng.random()
        if r < 0.45:
            toks = random_prompt(rng)
            try:
                want = ref.admit(toks)
            except ValueError:
                with pytest.raises(ValueError):
                    lib.admit(toks)
            else:
                assert lib.admit(toks) == want, (step, toks[:3], len(toks))
                jobs.append(want[0])
        elif r < 0.72 and jobs:
            pages = jobs.pop(int(rng.integers(0, len(jobs))))
            ref.release(pages)
            lib.release(pages)
        elif r < 0.82:
            n = int(rng.integers(0, 4))
            if n <= ref.allocatable():
                got = lib.alloc(n)
                assert got == ref.alloc(n)
                privs.append(got)
        elif r < 0.88 and privs:
            pages = privs[int(rng.integers(0, len(privs)))]
            ref.retain(pages)
            lib.retain(pages)
            privs.append(list(pages))
        elif r < 0.94 and privs:
            pages = privs.pop()
            ref.release(pages)
            lib.release(pages)
        else:
            mr = bool(rng.integers(0, 2))
            want = ref.defrag(mr)
            got = lib.defrag(mr)
            assert got[0] == want[0] and got[1] == [tuple(m) for m in want[1]], step
            jobs = [[want[0][p] for p in pages] for pages in jobs]
            privs = [[want[0][p] for p in pages] for pages in privs]
        assert tuple(lib.stats()) == ref.stats(), step


def test_same_tokens_at_another_position_do_not_match(pk):
    """A page is found by its whole prefix: page tokens that recur at another
    position, or after another prefix, are not a hit."""
    a = list(range(256)) + list(range(1000, 1256)) + [1]
    b = list(range(1000, 1256)) + [2]                # page 0 of b = page 1 of a
    c = list(range(5000, 5256)) + list(range(1000, 1256)) + [3]
    for pool in (opool.PagePool(12), Lib(pk, 12)):
        assert pool.admit(a)[1] == 0
        assert pool.admit(b)[1] == 0
        assert pool.admit(c)[1] == 0
        assert pool.admit(a + [4])[1] == 512


def test_error_paths_change_nothing(pk):
    pool = Lib(pk, 4)
    pages, _ = pool.admit(list(range(600)))
    before = pool.stats()
    with pytest.raises(pk.PkvError):
        pk.pkv_pool_release(pool.h, [pages[0], pages[0]])       # twice, referenced once
    with pytest.raises(pk.PkvError):
        pk.pkv_pool_retain(pool.h, [3])                         # FREE page
    with pytest.raises(pk.PkvError):
        pk.pkv_pool_alloc(pool.h, 2)                            # one page left
    with pytest.raises(pk.PkvError):
        pk.pkv_pool_admit(pool.h, list(range(600)), max_pages=2)
    with pytest.raises(pk.PkvError):
        pk.pkv_pool_admit(pool.h, list(range(2000, 2600)))      # three fresh pages, one left
    assert pool.stats() == before
    assert pk.LIB.pkv_pool_create(0) is None
    assert pk.LIB.pkv_pool_stats(None, None) == pk.PKV_ERR_NULL
