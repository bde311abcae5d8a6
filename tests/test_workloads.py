"""Input generators: determinism, layouts, bf16 rounding, the config-5 queue.
Runs on the CPU and keeps to small sizes."""

import numpy as np
import torch

from workloads import (f32_to_bf16_bits, bf16_bits_to_f32, BF16_QNAN, make_tiny_case,
                       make_accept_case, Config5Queue, kv_logical_bytes)
from workloads.configs import PAGE


def test_bf16_rounding_matches_torch_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.3895314e38,
                                  1e-40, -1e-40, np.inf, -np.inf], dtype=np.float32)])
    # exact ties at the bf16 boundary
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    assert f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == BF16_QNAN
    np.testing.assert_array_equal(bf16_bits_to_f32(ours[:100]),
                                  torch.from_numpy(x[:100]).to(torch.bfloat16).float().numpy())


def test_tiny_case_layout_and_determinism():
    a = make_tiny_case(3, [300, 5], [2, 1], Hq=4, Hkv=2, D=64, table_width=3)
    b = make_tiny_case(3, [300, 5], [2, 1], Hq=4, Hkv=2, D=64, table_width=3)
    np.testing.assert_array_equal(a.k_pool, b.k_pool)
    assert a.q.shape == (3, 4, 64) and a.k_pool.shape[1:] == (2, PAGE, 64)
    assert a.block_table.shape == (2, 3)
    assert (a.block_table[0, 2] == -1) and (a.block_table[1, 1:] == -1).all()
    used = set(a.block_table[0, :2]) | {a.block_table[1, 0]}
    assert len(used) == 3
    # tail of the last page and unreferenced pages are NaN, valid slots are not
    p_last = a.block_table[0, 1]
    assert (a.k_pool[p_last, :, 44:] == BF16_QNAN).all()
    assert not (a.k_pool[p_last, :, :44] == BF16_QNAN).any()
    spare = sorted(set(range(a.num_pages)) - used)
    assert (a.v_pool[spare] == BF16_QNAN).all()


def test_logical_bytes():
    assert kv_logical_bytes(np.array([300]), 2, 64) == 153600
    assert kv_logical_bytes(np.full(8, 8192), 8, 128) == 268435456


def test_accept_case_packing():
    c = make_accept_case(1, [6, 1, 3], 500)
    assert c.logits.shape == (10, 500)
    assert list(c.n_draft) == [5, 0, 2]
    assert c.draft_ids.shape == (7,)
    assert ((0 <= c.planted_match) & (c.planted_match <= c.n_draft)).all()
    assert ((0 <= c.draft_ids) & (c.draft_ids < 500)).all()


def test_config5_queue_is_a_valid_fifo_over_the_pool():
    q = Config5Queue(seed=0, n_jobs=12, D=64, Hq=4, Hkv=2, vocab=64)
    ghosts = set(q.ghost_pages)
    assert 0 < len(ghosts) <= 64
    seen = []
    for st in q.steps():
        c = st.case
        pages = []
        for b in range(c.num_seqs):
            n = -(-int(c.seq_lens[b]) // PAGE)
            pages += list(c.block_table[b, :n])
        assert len(pages) == len(set(pages)), "a page serves two live jobs"
        assert not (set(pages) & ghosts), "a job landed on a ghost page"
        assert all(0 <= p < 256 for p in pages)
        assert c.total_q == int(c.q_lens.sum())
        assert st.accept.total_rows == c.total_q
        seen.append(st.job_ids[0])
    assert seen == list(range(12))     # the oldest job retires each step
