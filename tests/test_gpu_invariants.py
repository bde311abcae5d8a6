"""GPU invariants, compared bit-exact with the GPU's own output: the layout of
pages in the pool (contiguous, permuted, deduplicated or duplicated) and the
contents of everything a sequence does not reference never change a result;
repeated calls give identical bits; broken contracts raise an error flag
instead of faulting."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
from workloads import make_tiny_case, contiguous_twin, permute_pages, duplicate_shared_pages, AttnCase
from tests.gpu_util import say, attn_gpu, DeviceCase, dev_bf16, assert_close


@pytest.fixture(scope="module")
def pk():
    import torch
    assert torch.cuda.is_available()
    import paged_kv_attention_attn_amd as pk
    return pk


CASES = [
    dict(seq_lens=[300, 1024, 77, 2000], q_lens=[1, 1, 1, 1], Hq=32, Hkv=8, D=128),
    dict(seq_lens=[600, 1000, 9], q_lens=[6, 3, 1], Hq=8, Hkv=2, D=128),
    dict(seq_lens=[520, 300], q_lens=[7, 2], Hq=8, Hkv=2, D=64),
]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_layout_invariance_is_bit_exact(pk, i):
    say(f"invariance case {i}")
    case = make_tiny_case(200 + i, num_pages=sum(-(-s // 256) for s in CASES[i]["seq_lens"]) + 5,
                          table_width=12, **CASES[i])
    base, f0 = attn_gpu(case, pk)
    assert f0 == 0
    for name, other in (("contiguous", contiguous_twin(case)), ("permuted", permute_pages(case, 1)),
                        ("permuted2", permute_pages(case, 2)), ("duplicated", duplicate_shared_pages(case))):
        got, f = attn_gpu(other, pk)
        assert f == 0
        np.testing.assert_array_equal(base, got, err_msg=name)


def test_shared_prefix_equals_private_copies(pk):
    rng = np.random.default_rng(3)
    case = make_tiny_case(300, [256 * 6 + 10] + [256 * 6 + int(x) for x in rng.integers(1, 256, 7)],
                          [1, 2, 1, 6, 1, 1, 3, 1], Hq=32, Hkv=8, D=128, num_pages=80, table_width=7)
    # make every sequence share the first 6 pages of sequence 0
    case.block_table[1:, :6] = case.block_table[0, :6]
    base, f0 = attn_gpu(case, pk)
    assert f0 == 0
    got, f1 = attn_gpu(duplicate_shared_pages(case), pk)
    assert f1 == 0
    np.testing.assert_array_equal(base, got)


def test_unreferenced_contents_and_spare_entries_do_not_matter(pk):
    kw = dict(Hq=8, Hkv=2, D=128, num_pages=20, table_width=10)
    clean = make_tiny_case(301, [300, 1000, 600], [1, 6, 3], poison=False, **kw)
    poisoned = make_tiny_case(301, [300, 1000, 600], [1, 6, 3], poison=True, **kw)
    poisoned.block_table[0, 2:] = [5, 10 ** 6, -3, 19, 0, 7, 7, 1]      # garbage past the last page
    poisoned.block_table[2, 3:] = -(10 ** 6)
    a, fa = attn_gpu(clean, pk)
    b, fb = attn_gpu(poisoned, pk)
    assert fa == 0 and fb == 0
    assert np.all(np.isfinite(b))
    np.testing.assert_array_equal(a, b)


def test_repeated_calls_are_identical(pk):
    import torch
    case = make_tiny_case(302, [3000, 700, 4100], [5, 1, 2], Hq=8, Hkv=2, D=128)
    dc = DeviceCase(case, pk)
    first = dc.result()
    for _ in range(3):
        dc.run()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(first, dc.out.cpu().numpy())
    assert dc.errors() == 0


def test_broken_contracts_set_flags_without_faulting(pk):
    import torch
    case = make_tiny_case(303, [600, 300], [1, 1], Hq=8, Hkv=2, D=64, num_pages=8)
    say("out-of-range page index")
    bad = AttnCase("badpage", case.q, case.k_pool, case.v_pool, case.block_table.copy(), case.seq_lens,
                   case.q_lens, case.scale)
    bad.block_table[0, 1] = 8            # == num_pages
    dc = DeviceCase(bad, pk)
    dc.run()
    torch.cuda.synchronize()
    assert dc.errors() & pk.PKV_EFLAG_PAGE
    say("window longer than max_q_len")
    bad2 = AttnCase("badq", np.concatenate([case.q, case.q]), case.k_pool, case.v_pool, case.block_table,
                    case.seq_lens, np.array([3, 1], np.int32), case.scale)
    dc2 = DeviceCase(bad2, pk, max_q_len=2)
    dc2.run()
    torch.cuda.synchronize()
    assert dc2.errors() & pk.PKV_EFLAG_QLEN
    say("sum(q_lens) beyond total_q")
    bad3 = AttnCase("badrows", case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens,
                    np.array([1, 2], np.int32), case.scale)
    dc3 = DeviceCase(bad3, pk, max_q_len=2)
    dc3.run()
    torch.cuda.synchronize()
    assert dc3.errors() & pk.PKV_EFLAG_ROWS


def sentinel_run(pk, case, total_q, max_q_len):
    """Attention with out pre-filled with a sentinel; returns (out, flags)."""
    import torch
    dc = DeviceCase(case, pk, max_q_len=max_q_len)
    if total_q != case.q.shape[0]:   # the call's row count, independent of q_lens
        q = np.zeros((total_q,) + case.q.shape[1:], case.q.dtype)
        n = min(total_q, case.q.shape[0])
        q[:n] = case.q[:n]
        dc.q = dev_bf16(q)
        dc.shape = pk.attn_shape(dc.q, dc.k, dc.bt, max_q_len, case.scale, 0)
        dc.ws = pk.new_attn_workspace(dc.shape)
        dc.out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dc.out.fill_(1234.5)
    dc.run()
    torch.cuda.synchronize()
    return dc.out.cpu().numpy(), dc.errors()


@pytest.mark.parametrize("max_q_len", [2, 40])   # the split kernel; the long-window kernel (rows > 64)
def test_negative_q_len_is_flagged_and_later_rows_are_left_alone(pk, max_q_len):
    say(f"q_lens (2, -1, 2): QLEN flagged, max_q_len {max_q_len}")
    case = make_tiny_case(304, [600, 300, 500], [2, 1, 2], Hq=8, Hkv=2, D=64)
    ref = oracle.attention(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens, case.q_lens,
                           case.scale)
    bad = AttnCase("negq", case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens,
                   np.array([2, -1, 2], np.int32), case.scale)
    got, flags = sentinel_run(pk, bad, case.q.shape[0], max_q_len)
    assert flags & pk.PKV_EFLAG_QLEN
    assert_close(got[:2], ref[:2], "sequence 0, before the negative length")
    # sequence 2's rows would start at row 1 by the prefix sum: it is skipped, nothing else is written
    assert np.all(got[2:] == np.float32(1234.5))


@pytest.mark.parametrize("max_q_len", [2, 40])
def test_row_sum_below_total_q_is_flagged(pk, max_q_len):
    say(f"sum(q_lens) 3 < total_q 5: ROWS flagged, rows computed, the rest untouched, max_q_len {max_q_len}")
    case = make_tiny_case(305, [600, 300], [2, 1], Hq=8, Hkv=2, D=64)
    ref = oracle.attention(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens, case.q_lens,
                           case.scale)
    got, flags = sentinel_run(pk, case, 5, max_q_len)
    assert flags & pk.PKV_EFLAG_ROWS
    assert_close(got[:3], ref, "the rows q_lens covers")
    assert np.all(got[3:] == np.float32(1234.5))
