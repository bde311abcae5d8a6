"""GPU parity of the shared-prefix call (pkv_attn_fwd_shared): a batch whose
tables all begin with the same pages attends to them once for every window
row, then to each sequence's own tail, merged by log-sum-exp. Compared with
the oracle (which knows nothing of the sharing), on the prefix-dedup
configuration and on small decode, verify and tail-prefill shapes; plus its
contract flags and repeated calls on one workspace."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
from workloads import make_config, normal_bf16, AttnCase, BF16_QNAN
from tests.gpu_util import say, assert_close, dev_bf16, dev_i32


@pytest.fixture(scope="module")
def pk():
    import torch
    assert torch.cuda.is_available()
    import paged_kv_attention_attn_amd as pk
    return pk


def run_shared(pk, case, shared_pages, max_q_len=None):
    import torch
    q, k, v = dev_bf16(case.q), dev_bf16(case.k_pool), dev_bf16(case.v_pool)
    bt, sl, ql = dev_i32(case.block_table), dev_i32(case.seq_lens), dev_i32(case.q_lens)
    mq = max_q_len if max_q_len is not None else int(case.q_lens.max())
    shape = pk.attn_shape(q, k, bt, mq, case.scale)
    ws = pk.new_attn_shared_workspace(shape, shared_pages)
    out = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    pk.pkv_attn_fwd_shared(q, k, v, bt, sl, ql, out, shape, shared_pages, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    out.fill_(float("nan"))
    pk.pkv_attn_fwd_shared(q, k, v, bt, sl, ql, out, shape, shared_pages, ws)   # the workspace is reusable
    torch.cuda.synchronize()
    again = out.cpu().numpy()
    return got, again, pk.pkv_attn_check_errors(ws)


def shared_case(seed, shared_pages, tails, q_lens, Hq=8, Hkv=2, D=128, spare=3):
    """Sequences whose tables start with the same shared_pages pages; each has
    tails[b] more tokens in private pages. Unreferenced pages and tails past
    the lengths are NaN."""
    rng = np.random.default_rng(seed)
    B = len(tails)
    own = [-(-int(t) // 256) for t in tails]
    P = shared_pages + sum(own) + spare
    perm = rng.permutation(P).astype(np.int32)
    W = shared_pages + max(own) + 1
    table = np.full((B, W), -1, np.int32)
    table[:, :shared_pages] = perm[:shared_pages]
    o = shared_pages
    for b in range(B):
        table[b, shared_pages:shared_pages + own[b]] = perm[o:o + own[b]]
        o += own[b]
    seq_lens = (shared_pages * 256 + np.asarray(tails)).astype(np.int32)
    q_lens = np.asarray(q_lens, np.int32)
    k = normal_bf16(rng, (P, Hkv, 256, D))
    v = normal_bf16(rng, (P, Hkv, 256, D))
    used = set(table[table >= 0].tolist())
    for p in range(P):
        if p not in used:
            k[p] = BF16_QNAN
            v[p] = BF16_QNAN
    for b in range(B):
        last, fill = int(table[b, shared_pages + own[b] - 1]), int(tails[b]) % 256
        if fill:
            k[last, :, fill:] = BF16_QNAN
            v[last, :, fill:] = BF16_QNAN
    q = normal_bf16(rng, (int(q_lens.sum()), Hq, D))
    return AttnCase("shared", q, k, v, table, seq_lens, q_lens, float(np.float32(1 / np.sqrt(D))))


def oracle_attn(case):
    return oracle.attention(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens, case.q_lens,
                            case.scale)


SHAPES = [
    # shared_pages, tails, q_lens, Hq, Hkv, D
    (1, [1, 100, 256, 257, 600], [1, 1, 1, 1, 1], 8, 2, 128),     # decode, tails across page ends
    (3, [6, 40, 300], [6, 3, 6], 32, 8, 128),                    # verify windows (24 rows), 8 KV heads
    (2, [16, 500, 77, 1000], [16, 2, 9, 1], 8, 2, 64),           # 64 rows, head_dim 64
    (5, [10] * 70, [1] * 70, 8, 8, 128),                         # one KV head per q head, 70 sequences
    # windows past the decode / verify kernel: the tails go through the
    # long-window kernel with the shared pages skipped
    (2, [300, 40, 600], [300, 20, 150], 8, 2, 128),              # tail prefills (q_len <= tail)
    (1, [256, 5, 700, 33], [256, 5, 700, 33], 8, 2, 64),         # every tail token a window row
    (3, [100, 1, 500], [100, 1, 3], 32, 8, 128),                 # long, decode and verify windows mixed
    # 2200 stacked rows per KV head: too many for the decode / verify row
    # tile, so the 256-row shared tiles over 3 key splits, then the merge kernel
    (2, [200, 150, 100, 100], [200, 150, 100, 100], 32, 8, 128),
    # 8192 stacked rows per KV head: 256 row tiles, so a single key split,
    # merged into the tails' rows inside the shared kernel
    (2, [256] * 8, [256] * 8, 32, 8, 128),
]


@pytest.mark.parametrize("i", range(len(SHAPES)))
def test_shared_prefix_matches_the_oracle(pk, i):
    sp, tails, q_lens, Hq, Hkv, D = SHAPES[i]
    say(f"shared prefix {i}: {sp} pages, tails {tails[:6]}, q_lens {q_lens[:6]}, Hq {Hq} Hkv {Hkv} D {D}")
    case = shared_case(400 + i, sp, tails, q_lens, Hq, Hkv, D)
    got, again, flags = run_shared(pk, case, sp)
    assert flags == 0
    assert_close(got, oracle_attn(case), f"shared {i}")
    assert np.array_equal(got, again), "repeated call differs"


def test_dedup_configuration(pk):
    """The prefix-dedup configuration: 100 sequences sharing 16 pages."""
    say("shared prefix: dedup configuration (100 x 16 shared pages)")
    case, _ = make_config(4)
    got, again, flags = run_shared(pk, case, 16)
    assert flags == 0
    assert_close(got, oracle_attn(case), "dedup shared")
    assert np.array_equal(got, again)


def test_dedup_tail_prefill_through_the_shared_call(pk):
    """The dedup prefill workload (100 tails of 1..256 tokens, every tail token
    a window row, over the 16 shared pages) through the shared call: sampled
    rows against the oracle, repeated calls bit-identical."""
    from workloads import make_prefill_config
    from tests.test_gpu_prefill import sample_picks, check_sampled
    say("shared prefix: dedup tail prefill, 100 tails over 16 shared pages")
    case = make_prefill_config("dedup")
    got, again, flags = run_shared(pk, case, 16)
    assert flags == 0
    check_sampled(case, got, sample_picks(case, np.random.default_rng(8), 40), "shared dedup prefill")
    assert np.array_equal(got, again), "repeated call differs"


def test_zero_shared_pages_is_the_plain_call(pk):
    case = shared_case(420, 2, [30, 300], [2, 1])
    got, _, flags = run_shared(pk, case, 0)
    assert flags == 0
    assert_close(got, oracle_attn(case), "shared 0")


def test_broken_contract_is_flagged(pk):
    say("shared prefix: contract checks")
    case = shared_case(421, 2, [30, 300, 50], [1, 1, 1])
    bad = AttnCase("bad", case.q, case.k_pool, case.v_pool, case.block_table.copy(), case.seq_lens,
                   case.q_lens, case.scale)
    bad.block_table[2, 1] = bad.block_table[2, 2]          # sequence 2 does not share page 1
    _, _, flags = run_shared(pk, bad, 2)
    assert flags & pk.PKV_EFLAG_PAGE
    short = AttnCase("short", case.q[:2], case.k_pool, case.v_pool, case.block_table[:2].copy(),
                     np.array([2 * 256 + 30, 2 * 256 + 300], np.int32), np.array([1, 1], np.int32), case.scale)
    short.seq_lens[0] = 2 * 256                              # no tail token: the window row is shared
    _, _, flags = run_shared(pk, short, 2)
    assert flags & pk.PKV_EFLAG_QLEN


def test_host_helper_finds_the_shared_prefix(pk):
    """pkv_shared_prefix_pages on the dedup configuration's host tables gives
    its 16 shared pages, and the call with that count matches the oracle."""
    case, _ = make_config(4)
    import torch
    shape = pk.attn_shape(dev_bf16(case.q), dev_bf16(case.k_pool), dev_i32(case.block_table), 1, case.scale)
    n = pk.pkv_shared_prefix_pages(case.block_table, case.seq_lens, case.q_lens, shape)
    assert n == 16
    got, _, flags = run_shared(pk, case, n)
    assert flags == 0
    assert_close(got, oracle_attn(case), "dedup via the helper")


def test_planned_shape_on_the_shared_call(pk):
    """A shape carrying a host plan (page count and split length for whole
    rows) on the shared-prefix call with the count the host helper derives:
    the tails plan their own splits, and the result matches the oracle."""
    import torch
    case = shared_case(430, 4, [10, 900, 3000, 256, 1], [1, 3, 2, 1, 4])
    q, k, v = dev_bf16(case.q), dev_bf16(case.k_pool), dev_bf16(case.v_pool)
    bt, sl, ql = dev_i32(case.block_table), dev_i32(case.seq_lens), dev_i32(case.q_lens)
    shape = pk.pkv_attn_plan(pk.attn_shape(q, k, bt, 4, case.scale), case.seq_lens)
    assert shape.pages_per_split > 0
    # the tables share 4 pages, but the last sequence (1025 tokens, a 4-row
    # window) has a window row that sees only 1021 keys: 3 pages are shared
    # by every row, the 4th goes with the tails
    n = pk.pkv_shared_prefix_pages(case.block_table, case.seq_lens, case.q_lens, shape)
    assert n == 3
    ws = pk.new_attn_shared_workspace(shape, n)
    out = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    pk.pkv_attn_fwd_shared(q, k, v, bt, sl, ql, out, shape, n, ws)
    torch.cuda.synchronize()
    assert pk.pkv_attn_check_errors(ws) == 0
    assert_close(out.cpu().numpy(), oracle_attn(case), "shared with a planned shape")


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.6])
@pytest.mark.parametrize("rows", ["few", "many"])
def test_shared_prefix_any_finite_scale(pk, scale, rows):
    """Any finite scale on both shared-prefix engines: the decode / verify
    row tile (few stacked rows, 24 here) takes the scale as given; the
    256-row tiles (many rows, 2200 per KV head here) run a negative scale on
    -q and a zero scale on q = 0; the tails and the merge take it as given."""
    if rows == "few":
        case, sp = shared_case(440, 2, [30, 300, 600], [1, 3, 2]), 2
    else:
        case, sp = shared_case(441, 2, [200, 150, 100, 100], [200, 150, 100, 100], 32, 8, 128), 2
    say(f"shared prefix, scale {scale}, {rows} rows")
    case = AttnCase("shared-scale", case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens,
                    case.q_lens, float(np.float32(scale)))
    got, again, flags = run_shared(pk, case, sp)
    assert flags == 0
    assert_close(got, oracle_attn(case), f"shared scale {scale} ({rows} rows)")
