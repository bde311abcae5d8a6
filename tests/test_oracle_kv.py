"""Pins for the K/V append and rollback oracle: a hand-derived worked example,
the gathered cache against an independent token-by-token picture of what it
must hold, page conservation, and the identities append + full accept and
append + empty accept. Runs on the CPU."""

import numpy as np
import pytest

from oracle import kv_cache as kv
from oracle.paged_attention import gather_sequence
from tests.fixtures import load_golden

WORKED = load_golden("kv_worked.json")
PAGE = 256


def _worked_inputs(Hkv=2, D=4):
    c = WORKED
    P = c["num_pages"]
    rng = np.random.default_rng(0)
    kp = rng.integers(0, 2**16, (P, Hkv, PAGE, D), dtype=np.uint16)
    vp = rng.integers(0, 2**16, (P, Hkv, PAGE, D), dtype=np.uint16)
    tq = sum(c["q_lens"])
    kn = (np.arange(tq * Hkv * D, dtype=np.uint16) + 1000).reshape(tq, Hkv, D)
    vn = kn + np.uint16(20000)
    free = np.full(P, -1, np.int32)
    free[:len(c["free_pages"])] = c["free_pages"]
    return kp, vp, np.array(c["table"], np.int32), np.array(c["seq_lens"], np.int32), \
        np.array(c["q_lens"], np.int32), kn, vn, free, len(c["free_pages"])


def test_worked_example():
    kp, vp, table, lens, ql, kn, vn, free, cnt = _worked_inputs()
    k2, v2, t2, l2, f2, c2 = kv.append(kp, vp, table, lens, ql, kn, vn, free, cnt)
    a = WORKED["after_append"]
    np.testing.assert_array_equal(t2, a["table"])
    np.testing.assert_array_equal(l2, a["seq_lens"])
    assert c2 == a["free_count"]
    row0 = [0, WORKED["q_lens"][0]]
    for b, i, page, slot in a["placements"]:
        np.testing.assert_array_equal(k2[page, :, slot], kn[row0[b] + i])
        np.testing.assert_array_equal(v2[page, :, slot], vn[row0[b] + i])
    t3, l3, f3, c3 = kv.rollback(t2, l2, ql, WORKED["accepted"], f2, c2)
    r = WORKED["after_rollback"]
    np.testing.assert_array_equal(t3, r["table"])
    np.testing.assert_array_equal(l3, r["seq_lens"])
    assert c3 == r["free_count"]
    np.testing.assert_array_equal(f3[:c3], r["free_top"])


def random_state(seed, B=5, P=40, W=6, Hkv=2, D=8, max_q=7):
    """Tables that partition some pages of the pool, the rest free (shuffled)."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(P).astype(np.int32)
    lens = rng.integers(0, (W - 1) * PAGE, B)
    lens[0] = 2 * PAGE                       # a length on a page boundary
    ql = rng.integers(0, max_q + 1, B)
    ql[0] = max(ql[0], 1)
    table = np.full((B, W), -1, np.int32)
    used = 0
    for b in range(B):
        n = -(-int(lens[b]) // PAGE)
        table[b, :n] = perm[used:used + n]
        used += n
    free = np.full(P, -1, np.int32)
    free[:P - used] = perm[used:]
    kp = rng.integers(0, 2**16, (P, Hkv, PAGE, D), dtype=np.uint16)
    vp = rng.integers(0, 2**16, (P, Hkv, PAGE, D), dtype=np.uint16)
    tq = int(ql.sum())
    kn = rng.integers(0, 2**16, (tq, Hkv, D), dtype=np.uint16)
    vn = rng.integers(0, 2**16, (tq, Hkv, D), dtype=np.uint16)
    return kp, vp, table, lens.astype(np.int32), ql.astype(np.int32), kn, vn, free, P - used


def logical_cache(kp, table, lens):
    """Token-by-token picture of each sequence: position -> [Hkv, D] bits,
    read slot by slot (independent of gather_sequence's page reshaping)."""
    out = []
    for b in range(table.shape[0]):
        seq = []
        for pos in range(int(lens[b])):
            seq.append(kp[table[b, pos // PAGE], :, pos % PAGE, :].copy())
        out.append(seq)
    return out


def referenced(table, lens):
    pages = []
    for b in range(table.shape[0]):
        pages += list(table[b, :-(-int(lens[b]) // PAGE)])
    return pages


@pytest.mark.parametrize("seed", range(6))
def test_append_extends_every_sequence_by_its_window(seed):
    kp, vp, table, lens, ql, kn, vn, free, cnt = random_state(seed)
    before_k = logical_cache(kp, table, lens)
    before_v = logical_cache(vp, table, lens)
    k2, v2, t2, l2, f2, c2 = kv.append(kp, vp, table, lens, ql, kn, vn, free, cnt)
    np.testing.assert_array_equal(l2, lens + ql)
    after_k, after_v = logical_cache(k2, t2, l2), logical_cache(v2, t2, l2)
    row = 0
    for b in range(len(lens)):
        exp_k = before_k[b] + [kn[row + i] for i in range(ql[b])]
        exp_v = before_v[b] + [vn[row + i] for i in range(ql[b])]
        row += ql[b]
        assert len(after_k[b]) == len(exp_k)
        for x, y in zip(after_k[b], exp_k):
            np.testing.assert_array_equal(x, y)
        for x, y in zip(after_v[b], exp_v):
            np.testing.assert_array_equal(x, y)
        # the same through the attention oracle's page gather
        g = gather_sequence(k2, t2[b], l2[b])
        np.testing.assert_array_equal(g.transpose(1, 0, 2), np.array(exp_k).reshape(-1, *kn.shape[1:]))
    # pages: exactly what the lengths need, no page both free and used, none lost
    for b in range(len(lens)):
        n = -(-int(l2[b]) // PAGE)
        assert np.all(t2[b, :n] >= 0) and np.all(t2[b, n:] == -1)
    used = referenced(t2, l2)
    assert len(set(used)) == len(used)
    assert sorted(used + list(f2[:c2])) == list(range(kp.shape[0]))
    # nothing outside the written slots changed
    changed = np.argwhere(np.any(k2 != kp, axis=(1, 3)))
    for page, slot in changed:
        assert any(page == t2[b, pos // PAGE] and slot == pos % PAGE
                   for b in range(len(lens)) for pos in range(lens[b], l2[b]))


@pytest.mark.parametrize("seed", range(6))
def test_rollback_keeps_the_accepted_prefix(seed):
    kp, vp, table, lens, ql, kn, vn, free, cnt = random_state(seed + 10)
    k2, v2, t2, l2, f2, c2 = kv.append(kp, vp, table, lens, ql, kn, vn, free, cnt)
    rng = np.random.default_rng(seed)
    acc = np.array([rng.integers(0, q + 1) for q in ql], np.int32)
    t3, l3, f3, c3 = kv.rollback(t2, l2, ql, acc, f2, c2)
    np.testing.assert_array_equal(l3, lens + acc)
    before, after2, after3 = logical_cache(kp, table, lens), logical_cache(k2, t2, l2), logical_cache(k2, t3, l3)
    for b in range(len(lens)):
        assert len(after3[b]) == lens[b] + acc[b]
        for x, y in zip(after3[b], after2[b][:lens[b] + acc[b]]):
            np.testing.assert_array_equal(x, y)
        n = -(-int(l3[b]) // PAGE)
        assert np.all(t3[b, :n] >= 0) and np.all(t3[b, n:] == -1)
    used = referenced(t3, l3)
    assert sorted(used + list(f3[:c3])) == list(range(kp.shape[0]))
    del before


@pytest.mark.parametrize("seed", range(4))
def test_full_accept_changes_nothing_and_empty_accept_undoes_the_append(seed):
    kp, vp, table, lens, ql, kn, vn, free, cnt = random_state(seed + 20)
    k2, v2, t2, l2, f2, c2 = kv.append(kp, vp, table, lens, ql, kn, vn, free, cnt)
    t3, l3, f3, c3 = kv.rollback(t2, l2, ql, ql, f2, c2)
    np.testing.assert_array_equal(t3, t2)
    np.testing.assert_array_equal(l3, l2)
    assert c3 == c2
    t4, l4, f4, c4 = kv.rollback(t2, l2, ql, np.zeros_like(ql), f2, c2)
    np.testing.assert_array_equal(t4, table)
    np.testing.assert_array_equal(l4, lens)
    assert c4 == cnt and sorted(f4[:c4]) == sorted(free[:cnt])


def test_released_pages_are_refilled_by_the_next_append():
    kp, vp, table, lens, ql, kn, vn, free, cnt = random_state(31)
    k2, v2, t2, l2, f2, c2 = kv.append(kp, vp, table, lens, ql, kn, vn, free, cnt)
    t3, l3, f3, c3 = kv.rollback(t2, l2, ql, np.zeros_like(ql), f2, c2)
    released = set(f3[c2:c3])
    k4, v4, t4, l4, f4, c4 = kv.append(k2, v2, t3, l3, ql, kn, vn, f3, c3)
    newly = set(t4[t4 >= 0]) - set(t3[t3 >= 0])
    assert released and released <= newly


def test_broken_contracts_raise_and_change_nothing():
    kp, vp, table, lens, ql, kn, vn, free, cnt = random_state(41)
    snap = [a.copy() for a in (kp, vp, table, lens, free)]
    with pytest.raises(ValueError):
        kv.append(kp, vp, table, lens, ql, kn, vn, free, 0)      # no free pages
    bad = lens.copy()
    bad[1] = table.shape[1] * PAGE                                # table row full ...
    ql1 = ql.copy()
    ql1[1] = 1                                                    # ... and one more token
    rows = int(ql1.sum())
    with pytest.raises(ValueError):
        kv.append(kp, vp, table, bad, ql1, kn[:1].repeat(rows, 0), vn[:1].repeat(rows, 0), free, cnt)
    with pytest.raises(ValueError):
        kv.rollback(table, lens, ql, ql + 1, free, cnt)          # more accepted than drafted
    for a, s in zip((kp, vp, table, lens, free), snap):
        np.testing.assert_array_equal(a, s)
