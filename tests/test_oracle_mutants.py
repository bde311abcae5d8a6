"""The pins must catch plausible mistakes. Each mutant below re-creates one
oracle function with a single planted defect (on the CPU, in this process
only); the pin battery must fail for every one of them."""

import numpy as np
import pytest

import oracle
import oracle.paged_attention as pa
import oracle.greedy_accept as oa
from oracle.brute import attention_brute, accept_brute
from workloads import make_tiny_case, make_accept_case
from tests.fixtures import load_golden, golden_attention_case

GOLDEN = load_golden("attention_closed_form.json")["cases"]
WORKED = load_golden("accept_worked.json")["sequences"]


def _rows_factory(group_fn=None, last_shift=0, use_scale=True, score_from_v=False,
                  normalise=True):
    def rows(q_rows, K, V, q_len, seq_len, scale):
        ql, Hq, D = q_rows.shape
        Hkv = K.shape[0]
        out = np.empty((ql, Hq, D))
        for i in range(ql):
            last = seq_len - ql + i + last_shift
            for h in range(Hq):
                g = group_fn(h, Hq, Hkv) if group_fn else h // (Hq // Hkv)
                src = V if score_from_v else K
                s = (scale if use_scale else 1.0) * (src[g, :last + 1] @ q_rows[i, h])
                p = np.exp(s - s.max())
                if normalise:
                    p /= p.sum()
                out[i, h] = p @ V[g, :last + 1]
        return out
    return rows


ATTN_MUTANTS = {
    "head group h % Hkv": dict(group_fn=lambda h, Hq, Hkv: h % Hkv),
    "window one key short": dict(last_shift=-1),
    "window one key long": dict(last_shift=+1),
    "scale dropped": dict(use_scale=False),
    "scores from V": dict(score_from_v=True),
    "softmax not normalised": dict(normalise=False),
}


def _gather_reversed(pool_bits, table_row, seq_len):
    n = -(-int(seq_len) // 256)
    tiles = pool_bits[np.asarray(table_row[:n])[::-1]]
    return tiles.transpose(1, 0, 2, 3).reshape(tiles.shape[1], n * 256, -1)[:, :seq_len]


def _gather_slot_shift(pool_bits, table_row, seq_len):
    n = -(-int(seq_len) // 256) + 1
    rows = np.asarray(table_row[:n])
    rows = np.where(rows < 0, rows[0], rows)
    tiles = pool_bits[rows]
    seq = tiles.transpose(1, 0, 2, 3).reshape(tiles.shape[1], n * 256, -1)
    return seq[:, 1:seq_len + 1]


def _attention_pins_pass():
    """True when every attention pin passes."""
    for c in GOLDEN:
        case = golden_attention_case(c)
        try:
            got = oracle.attention(case.q, case.k_pool, case.v_pool, case.block_table,
                                   case.seq_lens, case.q_lens, case.scale)
        except (ValueError, IndexError):
            return False
        if not np.allclose(got, np.array(c["expected"]), rtol=0, atol=max(c["tol"], 1e-15)):
            return False
    for seed, (sl, ql, Hq, Hkv, D) in enumerate([([300], [3], 4, 2, 4), ([5, 260], [2, 1], 2, 1, 4)]):
        case = make_tiny_case(seed, sl, ql, Hq=Hq, Hkv=Hkv, D=D, poison=False)
        got = oracle.attention(case.q, case.k_pool, case.v_pool, case.block_table,
                               case.seq_lens, case.q_lens, case.scale)
        ref = np.array(attention_brute(case.q, case.k_pool, case.v_pool, case.block_table,
                                       case.seq_lens, case.q_lens, case.scale))
        if not np.allclose(got, ref, rtol=1e-12, atol=1e-13):
            return False
    return True


def test_unmodified_oracle_passes_the_battery():
    assert _attention_pins_pass()


@pytest.mark.parametrize("name", list(ATTN_MUTANTS))
def test_attention_mutant_is_caught(monkeypatch, name):
    monkeypatch.setattr(pa, "attention_rows", _rows_factory(**ATTN_MUTANTS[name]))
    assert not _attention_pins_pass()


@pytest.mark.parametrize("fn", [_gather_reversed, _gather_slot_shift])
def test_gather_mutant_is_caught(monkeypatch, fn):
    monkeypatch.setattr(pa, "gather_sequence", fn)
    assert not _attention_pins_pass()


def _accept_pins_pass():
    logits = np.concatenate([np.array(s["logits"], dtype=np.float32) for s in WORKED])
    drafts = np.concatenate([np.array(s["drafts"], dtype=np.int32) for s in WORKED]).astype(np.int32)
    nd = np.array([len(s["drafts"]) for s in WORKED], dtype=np.int32)
    acc, nxt, _ = oa.accept(logits, drafts, nd)
    if list(acc) != [s["accepted"] for s in WORKED] or list(nxt) != [s["next"] for s in WORKED]:
        return False
    case = make_accept_case(9, [6, 6, 3, 1], 300)
    acc, _, _ = oa.accept(case.logits, case.draft_ids, case.n_draft)
    if not np.array_equal(acc, case.planted_match + 1):
        return False
    for preds, drafts in [([1, 0, 1], [1, 1]), ([0, 0], [0]), ([2], [])]:
        lg = np.zeros((len(preds), 3), np.float32)
        lg[np.arange(len(preds)), preds] = 1
        a, n, _ = oa.accept(lg, np.array(drafts, np.int32), np.array([len(drafts)], np.int32))
        if (a[0], n[0]) != accept_brute(preds, drafts):
            return False
    return True


def test_unmodified_accept_passes_the_battery():
    assert _accept_pins_pass()


def _argmax_last_tie(x):
    x = np.asarray(x, dtype=np.float32)
    return (x.shape[1] - 1 - np.argmax(x[:, ::-1], axis=1)).astype(np.int64)


def _accept_no_plus_one(logits, draft_ids, n_draft):
    a, n, f = ORIG_ACCEPT(logits, draft_ids, n_draft)
    return a - 1, n, f


def _accept_next_shifted(logits, draft_ids, n_draft):
    a, n, f = ORIG_ACCEPT(logits, draft_ids, n_draft)
    pred = ORIG_ARGMAX(logits)
    starts = np.concatenate([[0], np.cumsum(np.asarray(n_draft) + 1)[:-1]])
    nxt = np.array([pred[min(s + m + 1, s + d)] for s, m, d in zip(starts, f, n_draft)], np.int32)
    return a, nxt, f


ORIG_ACCEPT = oa.accept
ORIG_ARGMAX = oa.argmax_rows


@pytest.mark.parametrize("attr,fn", [("argmax_rows", _argmax_last_tie),
                                     ("accept", _accept_no_plus_one),
                                     ("accept", _accept_next_shifted)])
def test_accept_mutant_is_caught(monkeypatch, attr, fn):
    monkeypatch.setattr(oa, attr, fn)
    assert not _accept_pins_pass()


# ---- K/V append and rollback: each mutant is the oracle's own source with one
# planted defect, swapped in for the pin battery of tests/test_oracle_kv.py.

import inspect
import oracle.kv_cache as kvc
import tests.test_oracle_kv as kvpins

KV_MUTANTS = {
    "slot one late": ("append", "page, slot = int(table[b, pos // PAGE]), pos % PAGE",
                      "page, slot = int(table[b, pos // PAGE]), (pos + 1) % PAGE"),
    "no page for a window ending on a boundary": ("append", "for j in range(_pages(L), _pages(L + n)):",
                                                  "for j in range(_pages(L), _pages(L + n - 1)):"),
    "rows of the first sequence for every sequence": ("append", "k_pool[page, :, slot, :] = k_new[row + i]",
                                                      "k_pool[page, :, slot, :] = k_new[i]"),
    "rollback keeps one token too many": ("rollback", "new_len = S - n + a", "new_len = min(S, S - n + a + 1)"),
    "rollback releases one page too many": ("rollback",
                                            "for j in range(_pages(new_len), _pages(S)):",
                                            "for j in range(max(0, _pages(new_len) - 1), _pages(S)):"),
}


def _kv_mutant(fn_name, old, new):
    src = inspect.getsource(getattr(kvc, fn_name))
    assert old in src, old
    ns = dict(vars(kvc))
    exec(compile(src.replace(old, new), f"<mutant {fn_name}>", "exec"), ns)
    return ns[fn_name]


def _kv_battery():
    kvpins.test_worked_example()
    for seed in range(6):
        kvpins.test_append_extends_every_sequence_by_its_window(seed)
        kvpins.test_rollback_keeps_the_accepted_prefix(seed)
    for seed in range(4):
        kvpins.test_full_accept_changes_nothing_and_empty_accept_undoes_the_append(seed)


@pytest.mark.parametrize("name", list(KV_MUTANTS))
def test_kv_mutant_is_caught(name, monkeypatch):
    fn_name, old, new = KV_MUTANTS[name]
    monkeypatch.setattr(kvc, fn_name, _kv_mutant(fn_name, old, new))
    with pytest.raises(Exception):
        _kv_battery()


def test_kv_battery_passes_on_the_oracle():
    _kv_battery()
