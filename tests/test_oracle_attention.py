"""Pins for the attention oracle: hand-derived closed forms, brute force on
tiny inputs, and the invariants the pages fix (paged = unpaged, page order and
placement do not matter, a shared page equals private copies, the window is
causal). Runs on the CPU."""

import math

import numpy as np
import pytest

import oracle
from oracle.brute import attention_brute
from workloads import (make_tiny_case, contiguous_twin, permute_pages, duplicate_shared_pages,
                       f32_to_bf16_bits, AttnCase, BF16_QNAN)
from tests.fixtures import load_golden, golden_attention_case


def run(case):
    return oracle.attention(case.q, case.k_pool, case.v_pool, case.block_table,
                            case.seq_lens, case.q_lens, case.scale)


GOLDEN = load_golden("attention_closed_form.json")["cases"]


@pytest.mark.parametrize("c", GOLDEN, ids=[c["name"] for c in GOLDEN])
def test_golden_closed_form(c):
    case = golden_attention_case(c)
    got = run(case)
    np.testing.assert_allclose(got, np.array(c["expected"], dtype=np.float64), rtol=0,
                               atol=max(c["tol"], 0.0))
    brute = np.array(attention_brute(case.q, case.k_pool, case.v_pool, case.block_table,
                                     case.seq_lens, case.q_lens, case.scale))
    np.testing.assert_allclose(brute, np.array(c["expected"]), rtol=0, atol=max(c["tol"], 1e-15))


TINY = [
    # seq_lens, q_lens, Hq, Hkv, D
    ([1], [1], 1, 1, 4),
    ([5, 9], [1, 3], 2, 1, 8),
    ([257, 3], [2, 1], 4, 2, 4),
    ([300], [4], 4, 2, 8),
    ([256, 512, 17], [1, 5, 2], 2, 2, 4),
]


@pytest.mark.parametrize("seq_lens,q_lens,Hq,Hkv,D", TINY)
def test_oracle_matches_brute_force(seq_lens, q_lens, Hq, Hkv, D):
    case = make_tiny_case(11, seq_lens, q_lens, Hq=Hq, Hkv=Hkv, D=D)
    got = run(case)
    ref = np.array(attention_brute(case.q, case.k_pool, case.v_pool, case.block_table,
                                   case.seq_lens, case.q_lens, case.scale))
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_head_dim_64_case_matches_brute_force():
    case = make_tiny_case(3, [260], [2], Hq=2, Hkv=1, D=64)
    got = run(case)
    ref = np.array(attention_brute(case.q, case.k_pool, case.v_pool, case.block_table,
                                   case.seq_lens, case.q_lens, case.scale))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_single_visible_token_returns_value_row():
    case = make_tiny_case(5, [1, 1], [1, 1], Hq=4, Hkv=2, D=16)
    got = run(case)
    for b in range(2):
        page = case.block_table[b, 0]
        for h in range(4):
            v0 = oracle.decode_bf16(case.v_pool[page, h // 2, 0])
            np.testing.assert_array_equal(got[b, h], v0)


def test_equal_keys_average_visible_values():
    case = make_tiny_case(6, [300], [3], Hq=2, Hkv=1, D=8)
    page0 = case.block_table[0, 0]
    page1 = case.block_table[0, 1]
    key = case.k_pool[page0, 0, 0].copy()
    case.k_pool[page0, 0, :] = key
    case.k_pool[page1, 0, :44] = key
    got = run(case)
    V = np.concatenate([oracle.decode_bf16(case.v_pool[page0, 0]),
                        oracle.decode_bf16(case.v_pool[page1, 0, :44])])
    for i in range(3):
        visible = 300 - 3 + i + 1
        np.testing.assert_allclose(got[i, 0], V[:visible].mean(axis=0), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(got[i, 1], V[:visible].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_query_aligned_with_one_key_picks_its_value():
    case = make_tiny_case(7, [40], [1], Hq=1, Hkv=1, D=8)
    page = case.block_table[0, 0]
    j = 17
    kj = oracle.decode_bf16(case.k_pool[page, 0, j])
    # q = c * k_j with a large c: score j exceeds every other by far
    case.q[0, 0] = f32_to_bf16_bits((64.0 * kj).astype(np.float32))
    case.k_pool[page, 0, :40] = f32_to_bf16_bits(
        (oracle.decode_bf16(case.k_pool[page, 0, :40]) * 0.125).astype(np.float32))
    case.k_pool[page, 0, j] = f32_to_bf16_bits(kj.astype(np.float32))
    got = run(case)
    np.testing.assert_allclose(got[0, 0], oracle.decode_bf16(case.v_pool[page, 0, j]), rtol=1e-9,
                               atol=1e-9)


def test_gqa_equals_mha_over_repeated_kv_heads():
    case = make_tiny_case(8, [70, 300], [2, 1], Hq=6, Hkv=2, D=8)
    group = 3
    mha = AttnCase("mha", case.q, np.repeat(case.k_pool, group, axis=1),
                   np.repeat(case.v_pool, group, axis=1), case.block_table, case.seq_lens,
                   case.q_lens, case.scale)
    np.testing.assert_array_equal(run(case), run(mha))


def test_paged_equals_contiguous_layout():
    case = make_tiny_case(9, [300, 513, 5], [1, 3, 2], Hq=4, Hkv=2, D=8)
    np.testing.assert_array_equal(run(case), run(contiguous_twin(case)))


def test_page_permutation_does_not_change_output():
    case = make_tiny_case(10, [300, 600, 44], [2, 1, 1], Hq=4, Hkv=2, D=8, num_pages=12)
    base = run(case)
    for s in range(3):
        np.testing.assert_array_equal(base, run(permute_pages(case, s)))


def test_shared_prefix_equals_private_copies():
    # 5 sequences sharing 2 prefix pages plus one private page each
    rng = np.random.default_rng(0)
    P, Hkv, D = 9, 2, 8
    k = f32_to_bf16_bits(rng.standard_normal((P, Hkv, 256, D), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((P, Hkv, 256, D), dtype=np.float32))
    table = np.array([[3, 7, 0], [3, 7, 1], [3, 7, 2], [3, 7, 4], [3, 7, 5]], dtype=np.int32)
    seq_lens = np.array([513, 600, 700, 768, 520], dtype=np.int32)
    q_lens = np.array([1, 2, 1, 3, 1], dtype=np.int32)
    q = f32_to_bf16_bits(rng.standard_normal((8, 4, D), dtype=np.float32))
    case = AttnCase("dedup", q, k, v, table, seq_lens, q_lens, float(np.float32(0.35)))
    np.testing.assert_array_equal(run(case), run(duplicate_shared_pages(case)))


def test_unreferenced_pages_tails_and_spare_entries_are_never_read():
    clean = make_tiny_case(12, [300, 70], [2, 1], Hq=4, Hkv=2, D=8, table_width=4, poison=False)
    dirty = make_tiny_case(12, [300, 70], [2, 1], Hq=4, Hkv=2, D=8, table_width=4, poison=True)
    # spare table entries hold garbage, out of range on purpose
    dirty.block_table[0, 2:] = [10 ** 6, -5]
    dirty.block_table[1, 1:] = [-1, 77, 3]
    a, b = run(clean), run(dirty)
    assert np.all(np.isfinite(b))
    np.testing.assert_array_equal(a, b)
    assert (dirty.k_pool == BF16_QNAN).any()


def test_window_row_equals_decode_on_truncated_sequence():
    """Row i of a q_len window equals a q_len = 1 decode whose sequence ends
    at that row's token (causal inside the window, bottom-right aligned)."""
    q_len = 6
    case = make_tiny_case(13, [258], [q_len], Hq=4, Hkv=2, D=8)
    full = run(case)
    for i in range(q_len):
        L = 258 - q_len + i + 1
        one = AttnCase("row", case.q[i:i + 1], case.k_pool, case.v_pool, case.block_table,
                       np.array([L], np.int32), np.array([1], np.int32), case.scale)
        np.testing.assert_array_equal(full[i], run(one)[0])


def test_chunked_softmax_merge_matches_one_shot():
    """The log-sum-exp merge of per-chunk partial results (running max m,
    sum l, unnormalised accumulator) equals the one-shot softmax."""
    rng = np.random.default_rng(1)
    s = rng.standard_normal(700) * 3
    v = rng.standard_normal((700, 5))
    p = np.exp(s - s.max())
    ref = (p / p.sum()) @ v
    for cuts in ([256, 512], [1, 2, 3, 699], [100, 356, 357, 600]):
        parts = np.split(np.arange(700), cuts)
        m = [s[ix].max() for ix in parts]
        l = [np.exp(s[ix] - mi).sum() for ix, mi in zip(parts, m)]
        acc = [np.exp(s[ix] - mi) @ v[ix] for ix, mi in zip(parts, m)]
        M = max(m)
        w = [math.exp(mi - M) for mi in m]
        out = sum(wi * ai for wi, ai in zip(w, acc)) / sum(wi * li for wi, li in zip(w, l))
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_rejects_out_of_range_table_entry():
    case = make_tiny_case(14, [300], [1], Hq=2, Hkv=1, D=4)
    case.block_table[0, 1] = case.num_pages
    with pytest.raises(ValueError):
        run(case)


def test_rejects_window_longer_than_sequence():
    case = make_tiny_case(15, [3], [1], Hq=2, Hkv=1, D=4)
    bad = AttnCase("bad", np.concatenate([case.q] * 4), case.k_pool, case.v_pool,
                   case.block_table, case.seq_lens, np.array([4], np.int32), case.scale)
    with pytest.raises(ValueError):
        run(bad)


# Long windows (prefill, or a prefill chunk over cached tokens) use the same
# definition: window row i sees keys 0 .. seq_len - q_len + i.

@pytest.mark.parametrize("seq_lens,q_lens,Hq,Hkv,D", [
    ([20], [20], 2, 1, 4),          # a whole prompt, no cached prefix
    ([290, 40], [33, 40], 4, 2, 4),  # a chunk over 257 cached tokens; a whole short prompt
])
def test_long_window_matches_brute_force(seq_lens, q_lens, Hq, Hkv, D):
    case = make_tiny_case(16, seq_lens, q_lens, Hq=Hq, Hkv=Hkv, D=D)
    got = run(case)
    ref = np.array(attention_brute(case.q, case.k_pool, case.v_pool, case.block_table,
                                   case.seq_lens, case.q_lens, case.scale))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_whole_prompt_equals_library_causal_attention():
    """With no cached prefix (q_len = seq_len) the window is ordinary causal
    self-attention; torch's CPU scaled_dot_product_attention(is_causal=True)
    in float64, over K/V heads repeated to the q heads, must agree."""
    import torch
    L, Hq, Hkv, D = 300, 8, 2, 16
    case = make_tiny_case(17, [L], [L], Hq=Hq, Hkv=Hkv, D=D)
    got = run(case)
    q = torch.from_numpy(oracle.decode_bf16(case.q)).permute(1, 0, 2)               # [Hq, L, D]
    K = oracle.decode_bf16(oracle.gather_sequence(case.k_pool, case.block_table[0], L))
    V = oracle.decode_bf16(oracle.gather_sequence(case.v_pool, case.block_table[0], L))
    k = torch.from_numpy(K).repeat_interleave(Hq // Hkv, dim=0)                      # [Hq, L, D]
    v = torch.from_numpy(V).repeat_interleave(Hq // Hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True,
                                                           scale=case.scale)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


def test_prefill_in_chunks_equals_whole_prompt():
    """Prefilling a prompt in chunks, each chunk's window attending to the
    tokens cached before it, gives the rows of the whole-prompt window."""
    L = 530
    case = make_tiny_case(18, [L], [L], Hq=4, Hkv=2, D=8)
    whole = run(case)
    for lo, hi in ((0, 100), (100, 256), (256, 257), (257, 530)):
        part = AttnCase("chunk", case.q[lo:hi], case.k_pool, case.v_pool, case.block_table,
                        np.array([hi], np.int32), np.array([hi - lo], np.int32), case.scale)
        np.testing.assert_array_equal(run(part), whole[lo:hi])


# ---- attention over pools of already-decoded values (the quantized caches)

def test_decoded_pools_single_visible_token_returns_its_decoded_value():
    from oracle import q8_cache
    case = make_tiny_case(8, [1, 1], [1, 1], Hq=4, Hkv=2, D=16)
    kc, ks = q8_cache.encode(case.k_pool)
    vc, vs = q8_cache.encode(case.v_pool)
    K, V = q8_cache.decode(kc, ks), q8_cache.decode(vc, vs)
    got = oracle.attention_decoded(case.q, K, V, case.block_table, case.seq_lens, case.q_lens, case.scale)
    for b in range(2):
        page = case.block_table[b, 0]
        for h in range(4):
            # one visible key: weight 1 on its value, code x scale exactly
            np.testing.assert_array_equal(got[b, h], vc[page, h // 2, 0].astype(np.float64) * float(vs[page, h // 2, 0]))


def test_decoded_pools_with_equal_keys_average_the_decoded_values():
    from oracle import q4_cache
    case = make_tiny_case(9, [300], [2], Hq=2, Hkv=1, D=8)
    page0, page1 = case.block_table[0, 0], case.block_table[0, 1]
    key = case.k_pool[page0, 0, 0].copy()
    case.k_pool[page0, 0, :] = key
    case.k_pool[page1, 0, :44] = key
    kc, ks = q4_cache.encode(case.k_pool)
    vc, vs = q4_cache.encode(case.v_pool)
    K, V = q4_cache.decode(kc, ks), q4_cache.decode(vc, vs)
    got = oracle.attention_decoded(case.q, K, V, case.block_table, case.seq_lens, case.q_lens, case.scale)
    codes = np.concatenate([q4_cache.unpack(vc[page0, 0]), q4_cache.unpack(vc[page1, 0, :44])]).astype(np.float64)
    scales = np.concatenate([vs[page0, 0], vs[page1, 0, :44]]).astype(np.float64)
    vals = codes * scales[:, None]
    for i in range(2):
        visible = 300 - 2 + i + 1
        np.testing.assert_allclose(got[i, 0], vals[:visible].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_decoded_bf16_pools_give_the_bf16_result():
    case = make_tiny_case(10, [700, 33], [3, 1], Hq=4, Hkv=2, D=16)
    got = oracle.attention_decoded(case.q, oracle.decode_bf16(case.k_pool), oracle.decode_bf16(case.v_pool),
                                   case.block_table, case.seq_lens, case.q_lens, case.scale)
    ref = np.array(attention_brute(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens,
                                   case.q_lens, case.scale))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
