"""GPU parity of long windows (prefill, or a prefill chunk over cached
tokens): more than 64 rows per (sequence, KV head) run the long-window kernel
behind the same pkv_attn_fwd. Small cases are compared with the whole oracle;
the full-size workloads on sampled rows (window row i of a sequence equals the
oracle's single-row attention over the sequence cut after that row's token),
plus bit-exact layout invariance and the error flags."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
from workloads import make_tiny_case, make_prefill_config, duplicate_shared_pages, permute_pages, AttnCase
from tests.gpu_util import say, attn_gpu, assert_close, DeviceCase


@pytest.fixture(scope="module")
def pk():
    import torch
    assert torch.cuda.is_available()
    import paged_kv_attention_attn_amd as pk
    return pk


def oracle_attn(case):
    return oracle.attention(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens,
                            case.q_lens, case.scale)


def oracle_rows(case, picks):
    """Oracle rows for (sequence b, window row i) picks: the single-row
    attention of that row over the sequence cut after its token."""
    starts = np.concatenate([[0], np.cumsum(case.q_lens)])
    out = {}
    for b in sorted({b for b, _ in picks}):
        L, ql = int(case.seq_lens[b]), int(case.q_lens[b])
        K = oracle.decode_bf16(oracle.gather_sequence(case.k_pool, case.block_table[b], L))
        V = oracle.decode_bf16(oracle.gather_sequence(case.v_pool, case.block_table[b], L))
        for bb, i in picks:
            if bb != b:
                continue
            last = L - ql + i
            r = int(starts[b]) + i
            qrow = oracle.decode_bf16(case.q[r:r + 1])
            out[(b, i)] = oracle.attention_rows(qrow, K[:, :last + 1], V[:, :last + 1], 1, last + 1,
                                                case.scale)[0]
    return out


# tiles are 256 rows: 256 / group window tokens
PREFILL = [
    # seq_lens, q_lens, Hq, Hkv, D
    ([300], [300], 8, 2, 128),                          # whole prompt: 5 tiles, the first one partial
    ([517, 321, 40], [17, 65, 40], 8, 2, 128),          # chunks over cached tokens; tiles across pages
    ([700, 1], [700, 1], 8, 2, 64),                     # head_dim 64; a one-token window in the batch
    ([520], [520], 2, 2, 128),                          # one KV head per q head: 256 tokens per tile
    ([333, 90], [333, 20], 16, 2, 128),                 # group 8: 32 tokens per tile
    ([400], [400], 10, 2, 64),                          # group 5: 51 tokens (255 rows) per tile
    ([1300, 600], [64, 0], 32, 8, 128),                 # exactly one tile; a skipped sequence
    ([2000, 513], [1, 17], 8, 2, 128),                  # 68 rows: the long-window kernel for both
]


@pytest.mark.parametrize("i", range(len(PREFILL)))
def test_long_windows_match_the_oracle(pk, i):
    seq_lens, q_lens, Hq, Hkv, D = PREFILL[i]
    say(f"prefill case {i}: seq_lens={seq_lens} q_lens={q_lens} Hq={Hq} Hkv={Hkv} D={D}")
    case = make_tiny_case(300 + i, seq_lens, q_lens, Hq=Hq, Hkv=Hkv, D=D)
    assert case.max_q_len * Hq // Hkv > pk.PKV_MAX_ROWS
    got, flags = attn_gpu(case, pk)
    assert flags == 0
    assert_close(got, oracle_attn(case), f"prefill {i}")


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.3, 0.5])
def test_any_finite_scale(pk, scale):
    """The long-window softmax runs on a positive scale (a negative one is
    applied to -q); zero gives the plain mean of the visible values. Scales
    0.3 and 0.5 on head_dim 64 (2.4x and 4x the usual 1/sqrt(64)) make rows
    peaky, where a few keys carry most of the weight and bf16 rounding of
    their P would not average out."""
    say(f"prefill scale {scale}")
    case = make_tiny_case(340, [400, 150], [200, 150], Hq=8, Hkv=2, D=64, scale=scale)
    got, flags = attn_gpu(case, pk)
    assert flags == 0
    assert_close(got, oracle_attn(case), f"prefill scale {scale}")


def test_layout_invariance_and_repeat_are_bit_exact(pk):
    say("prefill: permuted pool and repeated calls, bit-exact")
    case = make_tiny_case(320, [900, 600, 300], [900, 300, 70], Hq=8, Hkv=2, D=128, table_width=6)
    base, f0 = attn_gpu(case, pk)
    assert f0 == 0
    for seed in (1, 2):
        got, f = attn_gpu(permute_pages(case, seed), pk)
        assert f == 0 and np.array_equal(got, base), f"permutation {seed}"
    dc = DeviceCase(case, pk)
    first = dc.result()
    assert np.array_equal(dc.result(), first) and np.array_equal(first, base)


def sample_picks(case, rng, n):
    """Window rows to check: the first and last of every tile boundary region
    of a few sequences, plus random ones."""
    B = case.num_seqs
    picks = set()
    for b in rng.choice(B, size=min(B, 6), replace=False):
        ql = int(case.q_lens[b])
        for i in (0, ql - 1, ql // 2, max(0, ql - 64), max(0, ql - 65)):
            picks.add((int(b), int(i)))
    while len(picks) < n:
        b = int(rng.integers(0, B))
        if case.q_lens[b] > 0:
            picks.add((b, int(rng.integers(0, case.q_lens[b]))))
    return sorted(picks)


def check_sampled(case, got, picks, what):
    starts = np.concatenate([[0], np.cumsum(case.q_lens)])
    ref = oracle_rows(case, picks)
    for (b, i), o in ref.items():
        assert_close(got[int(starts[b]) + i], o, f"{what} seq {b} row {i}")


def test_dedup_tail_prefill_full_size(pk):
    """100 sequences over a shared 16-page prefix prefill their private tails
    (1..256 tokens): sampled rows against the oracle, and the shared layout
    against private copies of every page, bit-exact."""
    say("prefill dedup: 100 tails over a shared 4096-token prefix")
    case = make_prefill_config("dedup")
    got, flags = attn_gpu(case, pk)
    assert flags == 0
    check_sampled(case, got, sample_picks(case, np.random.default_rng(5), 40), "dedup prefill")
    twin, f2 = attn_gpu(duplicate_shared_pages(case), pk)
    assert f2 == 0 and np.array_equal(twin, got)


def test_whole_prompt_prefill_full_size(pk):
    """8 sequences x 8192 tokens, every token a window row (the verify
    workload's cache as a whole-prompt prefill): sampled rows."""
    say("prefill full: 8 x 8192 tokens")
    case = make_prefill_config("full")
    dc = DeviceCase(case, pk)
    got = dc.result()
    assert dc.errors() == 0
    check_sampled(case, got, sample_picks(case, np.random.default_rng(6), 24), "full prefill")


@pytest.mark.timeout(900)
def test_whole_prompt_prefill_one_head_group_in_full(pk):
    """8 x 8192 whole-prompt prefill: every one of the 8192 window rows of
    one (sequence, KV head), all heads of its group, against the oracle."""
    case = make_prefill_config("full")
    rng = np.random.default_rng(7)
    b, g = int(rng.integers(0, case.num_seqs)), int(rng.integers(0, case.k_pool.shape[1]))
    Hq, Hkv = case.q.shape[1], case.k_pool.shape[1]
    group = Hq // Hkv
    say(f"prefill full: every row of sequence {b}, KV head {g} ({group} q heads x 8192 rows)")
    dc = DeviceCase(case, pk)
    got = dc.result()
    assert dc.errors() == 0
    L, ql = int(case.seq_lens[b]), int(case.q_lens[b])
    r0 = int(np.sum(case.q_lens[:b]))
    K = oracle.decode_bf16(oracle.gather_sequence(case.k_pool, case.block_table[b], L))[g:g + 1]
    V = oracle.decode_bf16(oracle.gather_sequence(case.v_pool, case.block_table[b], L))[g:g + 1]
    heads = slice(g * group, (g + 1) * group)
    qrows = oracle.decode_bf16(case.q[r0:r0 + ql, heads])
    ref = oracle.attention_rows(qrows, K, V, ql, L, case.scale)
    assert_close(got[r0:r0 + ql, heads], ref, f"full prefill seq {b} KV head {g}")


def test_broken_contracts_set_flags(pk):
    say("prefill: broken contracts set flags, other sequences unaffected")
    case = make_tiny_case(330, [600, 500], [200, 300], Hq=8, Hkv=2, D=64, table_width=4)
    ref = oracle_attn(case)
    # a window longer than max_q_len
    dc = DeviceCase(case, pk, max_q_len=250)
    got = dc.result()
    assert dc.errors() & pk.PKV_EFLAG_QLEN
    assert_close(got[:200], ref[:200], "sequence 0 beside a too-long window")
    # a table entry outside the pool: flagged, other sequence still right
    bad = AttnCase("bad", case.q, case.k_pool, case.v_pool, case.block_table.copy(), case.seq_lens,
                   case.q_lens, case.scale)
    bad.block_table[1, 1] = case.num_pages + 3
    dc = DeviceCase(bad, pk)
    got = dc.result()
    assert dc.errors() & pk.PKV_EFLAG_PAGE
    assert_close(got[:200], ref[:200], "sequence 0 beside a bad table entry")
