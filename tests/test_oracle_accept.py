"""Pins for the argmax / accept / window oracle: hand-worked fixtures from the
assisted-generation loop, brute-force enumeration, explicit tie and NaN rows,
and the planted-draft structure of the generated workloads. Runs on the CPU."""

import itertools

import numpy as np
import pytest

import oracle
from oracle.brute import argmax_brute, accept_brute
from workloads import make_accept_case
from tests.fixtures import load_golden

WORKED = load_golden("accept_worked.json")
WINDOW = load_golden("window_rule.json")


def test_worked_accept_examples():
    seqs = WORKED["sequences"]
    logits = np.concatenate([np.array(s["logits"], dtype=np.float32) for s in seqs])
    drafts = np.concatenate([np.array(s["drafts"], dtype=np.int32) for s in seqs]).astype(np.int32)
    n_draft = np.array([len(s["drafts"]) for s in seqs], dtype=np.int32)
    pred = oracle.argmax_rows(logits)
    np.testing.assert_array_equal(pred, np.concatenate([s["argmax"] for s in seqs]))
    acc, nxt, first = oracle.accept(logits, drafts, n_draft)
    np.testing.assert_array_equal(acc, [s["accepted"] for s in seqs])
    np.testing.assert_array_equal(nxt, [s["next"] for s in seqs])
    np.testing.assert_array_equal(first, [s["first_mismatch"] for s in seqs])


@pytest.mark.parametrize("c", WINDOW["cases"], ids=lambda c: c["why"])
def test_window_rule_table(c):
    got = oracle.window_next([c["window"]], [c["n_draft"]], [c["accepted"]])
    assert int(got[0]) == c["next_window"]


def test_initial_window_is_five():
    assert WINDOW["initial_window"] == 5
    case = make_accept_case(0, [6, 6, 1], 50)
    assert list(case.window) == [5, 5, 5]


def test_argmax_matches_brute_force_on_random_rows():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((40, 37)).astype(np.float32)
    x[3, [4, 20]] = 9.0                      # a tie
    x[5, :] = -np.inf                        # all -inf: index 0
    x[6, 7] = np.nan                         # NaN wins
    x[7, [2, 30]] = np.nan                   # first NaN wins
    x[8, :] = 0.0
    x[8, 10] = -0.0                          # -0.0 == 0.0: lowest index
    x[9, 36] = np.inf
    x[10, [0, 36]] = np.inf
    got = oracle.argmax_rows(x)
    for r in range(40):
        assert got[r] == argmax_brute(x[r]), r


def test_argmax_stays_exact_in_float32():
    # adjacent float32 values must not be merged by any widening or rounding
    a = np.float32(1.0)
    b = np.nextafter(a, np.float32(2.0))
    row = np.array([[a, b, a]], dtype=np.float32)
    assert oracle.argmax_rows(row)[0] == 1


def test_accept_exhaustive_small_vocab():
    """Every prediction/draft combination for vocab <= 3 and n <= 3 drafts."""
    for V in (2, 3):
        for n in range(0, 4):
            for preds in itertools.product(range(V), repeat=n + 1):
                logits = np.zeros((n + 1, V), dtype=np.float32)
                logits[np.arange(n + 1), preds] = 1.0
                for drafts in itertools.product(range(V), repeat=n):
                    acc, nxt, first = oracle.accept(logits, np.array(drafts, np.int32),
                                                    np.array([n], np.int32))
                    ea, en = accept_brute(list(preds), list(drafts))
                    assert (acc[0], nxt[0]) == (ea, en)
                    assert first[0] == acc[0] - 1


def test_accept_on_planted_drafts_recovers_planted_prefix():
    q_lens = [6] * 8 + [1, 2, 3, 4, 5, 7, 16]
    case = make_accept_case(4, q_lens, 1000)
    acc, nxt, first = oracle.accept(case.logits, case.draft_ids, case.n_draft)
    np.testing.assert_array_equal(first, case.planted_match)
    np.testing.assert_array_equal(acc, case.planted_match + 1)
    # full match gives +2, anything else -1
    w = oracle.window_next(case.window, case.n_draft, acc)
    full = case.planted_match == case.n_draft
    np.testing.assert_array_equal(w, np.where(full, case.window + 2, case.window - 1))


def test_accept_rejects_inconsistent_packing():
    logits = np.zeros((3, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.accept(logits, np.zeros(1, np.int32), np.array([1], np.int32))
