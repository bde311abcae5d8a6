"""The C-ABI library: it loads, exports every function include/pkv.h declares,
and its host-side checks reject bad shapes before any GPU work. No kernel is
launched here, so these run on a machine without a GPU."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(pkv_[a-z_0-9]+)\s*\(", text,
                       flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def pk():
    import paged_kv_attention_attn_amd as pk
    return pk


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("pkv_attn_fwd", "pkv_accept", "pkv_attn_workspace_bytes",
                     "pkv_accept_workspace_bytes", "pkv_window_next", "pkv_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol(pk):
    lib = ctypes.CDLL(pk.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(pk.EXPORTS) == declared_functions()


def test_struct_layouts_match_the_header(pk):
    assert ctypes.sizeof(pk.pkv_attn_shape) == 48
    assert ctypes.sizeof(pk.pkv_accept_shape) == 16
    assert ctypes.sizeof(pk.pkv_kv_shape) == 28


def test_window_rule_on_the_host(pk):
    assert pk.pkv_window_next(5, 5, 6) == 7
    assert pk.pkv_window_next(5, 5, 3) == 4
    assert pk.pkv_window_next(1, 1, 1) == 1
    assert pk.pkv_window_next(3, 0, 1) == 5


def good_shape(pk, **kw):
    f = dict(num_seqs=4, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=256, num_pages=64,
             max_pages_per_seq=8, total_q=4, max_q_len=1, scale=0.088)
    f.update(kw)
    return pk.pkv_attn_shape(**f)


@pytest.mark.parametrize("bad", [
    dict(num_q_heads=30),            # Hq % Hkv != 0
    dict(head_dim=96),               # unsupported D
    dict(page_size=128),             # pages are 256 tokens
    dict(max_q_len=0),
    dict(max_q_len=8 * 256 + 1),          # longer than a table row can hold
    dict(num_q_heads=8 * 65),             # a head group wider than 64 rows
    dict(num_pages=0), dict(max_pages_per_seq=0), dict(num_seqs=-1),
    dict(scale=float("nan")),
    dict(total_pages=-1),                 # the planning hint counts pages
    dict(pages_per_split=-1), dict(pages_per_split=65),   # a split stages at most 64 table entries
    # long windows of 2^20 rows in a head group of 64: 2^31 query tiles, past the item bound
    dict(num_seqs=2**13, num_q_heads=64, num_kv_heads=1, max_pages_per_seq=2**16, max_q_len=2**20, total_q=1),
])
def test_bad_attention_shapes_are_rejected_before_launch(pk, bad):
    s = good_shape(pk, **bad)
    assert pk.pkv_attn_workspace_bytes(s) == 0
    rc = pk.LIB.pkv_attn_fwd(None, None, None, None, None, None, None, ctypes.byref(s), None, 0, None)
    assert rc == pk.PKV_ERR_SHAPE


@pytest.mark.parametrize("ok", [dict(max_q_len=16), dict(max_q_len=17), dict(max_q_len=8 * 256),
                                dict(num_q_heads=64, max_q_len=16), dict(num_q_heads=8 * 64, max_q_len=1)])
def test_long_windows_and_wide_groups_are_accepted(pk, ok):
    # more than 64 rows per (sequence, KV head) runs the long-window kernel
    assert pk.pkv_attn_workspace_bytes(good_shape(pk, **ok)) > 0


def test_null_pointers_and_small_workspace_are_rejected(pk):
    s = good_shape(pk)
    dummy = ctypes.c_void_p(0x1000)
    rc = pk.LIB.pkv_attn_fwd(None, dummy, dummy, dummy, dummy, dummy, dummy, ctypes.byref(s), dummy,
                             1 << 30, None)
    assert rc == pk.PKV_ERR_NULL
    need = pk.pkv_attn_workspace_bytes(s)
    assert need > 0
    rc = pk.LIB.pkv_attn_fwd(dummy, dummy, dummy, dummy, dummy, dummy, dummy, ctypes.byref(s), dummy,
                             need - 1, None)
    assert rc == pk.PKV_ERR_WORKSPACE
    rc = pk.LIB.pkv_attn_fwd(dummy, dummy, dummy, dummy, dummy, dummy, dummy, None, dummy, need, None)
    assert rc == pk.PKV_ERR_NULL


def test_empty_batch_is_a_no_op(pk):
    s = good_shape(pk, num_seqs=0, total_q=0)
    rc = pk.LIB.pkv_attn_fwd(None, None, None, None, None, None, None, ctypes.byref(s), None, 0, None)
    assert rc == pk.PKV_OK


@pytest.mark.parametrize("bad", [dict(vocab=0), dict(max_draft=16), dict(total_rows=1, num_seqs=2),
                                 dict(num_seqs=-1)])
def test_bad_accept_shapes_are_rejected(pk, bad):
    f = dict(num_seqs=2, vocab=100, total_rows=4, max_draft=3)
    f.update(bad)
    s = pk.pkv_accept_shape(**f)
    assert pk.pkv_accept_workspace_bytes(s) == 0
    rc = pk.LIB.pkv_accept(None, None, None, None, None, None, ctypes.byref(s), None, 0, None)
    assert rc == pk.PKV_ERR_SHAPE


def test_accept_workspace_and_nulls(pk):
    s = pk.pkv_accept_shape(8, 128256, 48, 5)
    need = pk.pkv_accept_workspace_bytes(s)
    # one 8-byte key per (row, chunk): 16 chunks of 8016 logits per row here
    assert need == 48 * 16 * 8
    dummy = ctypes.c_void_p(0x1000)
    rc = pk.LIB.pkv_accept(dummy, dummy, dummy, dummy, dummy, None, ctypes.byref(s), dummy, need - 1,
                           None)
    assert rc == pk.PKV_ERR_WORKSPACE
    rc = pk.LIB.pkv_accept(None, dummy, dummy, dummy, dummy, None, ctypes.byref(s), dummy, need, None)
    assert rc == pk.PKV_ERR_NULL


def test_status_strings(pk):
    for code in (0, -1, -2, -3, -4):
        assert pk.pkv_status_string(code)
    assert pk.pkv_version() >= 100


@pytest.mark.parametrize("bad", [dict(head_dim=96), dict(page_size=128), dict(num_pages=0),
                                 dict(max_pages_per_seq=0), dict(total_q=-1), dict(num_seqs=-1),
                                 dict(num_pages=1 << 24)])
def test_bad_cache_shapes_are_rejected(pk, bad):
    f = dict(num_seqs=4, num_kv_heads=8, head_dim=128, page_size=256, num_pages=256,
             max_pages_per_seq=32, total_q=24)
    f.update(bad)
    s = pk.pkv_kv_shape(**f)
    assert pk.pkv_kv_workspace_bytes(s) == 0
    rc = pk.LIB.pkv_kv_append(*([None] * 9), ctypes.byref(s), None, 0, None)
    assert rc == pk.PKV_ERR_SHAPE
    rc = pk.LIB.pkv_kv_rollback(*([None] * 6), ctypes.byref(s), None, 0, None)
    assert rc == pk.PKV_ERR_SHAPE


def test_cache_calls_check_pointers_and_workspace(pk):
    s = pk.pkv_kv_shape(4, 8, 128, 256, 256, 32, 24)
    need = pk.pkv_kv_workspace_bytes(s)
    assert need >= 256 + 24 * 4
    d = ctypes.c_void_p(0x1000)
    assert pk.LIB.pkv_kv_append(*([d] * 9), ctypes.byref(s), d, need - 1, None) == pk.PKV_ERR_WORKSPACE
    assert pk.LIB.pkv_kv_append(*([d] * 8), None, ctypes.byref(s), d, need, None) == pk.PKV_ERR_NULL
    assert pk.LIB.pkv_kv_rollback(*([d] * 6), ctypes.byref(s), d, need - 1, None) == pk.PKV_ERR_WORKSPACE
    assert pk.LIB.pkv_kv_rollback(d, d, d, None, d, d, ctypes.byref(s), d, need, None) == pk.PKV_ERR_NULL
    empty = pk.pkv_kv_shape(0, 8, 128, 256, 256, 32, 0)
    assert pk.LIB.pkv_kv_append(*([None] * 9), ctypes.byref(empty), None, 0, None) == pk.PKV_OK


def test_page_move_calls_check_shapes_and_pointers_before_any_launch(pk):
    d = ctypes.c_void_p(0x1000)
    L = pk.LIB
    assert L.pkv_pool_copy_pages(d, d, d, d, -1, 8, 2, 64, None, None) == pk.PKV_ERR_SHAPE
    assert L.pkv_pool_copy_pages(d, d, d, d, 1, 8, 2, 96, None, None) == pk.PKV_ERR_SHAPE
    assert L.pkv_pool_copy_pages(d, d, d, d, 1, 0, 2, 64, None, None) == pk.PKV_ERR_SHAPE
    assert L.pkv_pool_copy_pages(None, d, d, d, 1, 8, 2, 64, None, None) == pk.PKV_ERR_NULL
    assert L.pkv_pool_copy_pages(None, None, None, None, 0, 8, 2, 64, None, None) == pk.PKV_OK
    assert L.pkv_table_remap(d, -1, 4, d, 8, None, None) == pk.PKV_ERR_SHAPE
    assert L.pkv_table_remap(d, 2, 0, d, 8, None, None) == pk.PKV_ERR_SHAPE
    assert L.pkv_table_remap(None, 2, 4, d, 8, None, None) == pk.PKV_ERR_NULL
    assert L.pkv_table_remap(None, 0, 4, None, 8, None, None) == pk.PKV_OK


def test_allocator_calls_reject_null_and_bad_sizes(pk):
    L = pk.LIB
    assert L.pkv_pool_create(0) is None and L.pkv_pool_create(-5) is None
    assert L.pkv_pool_create((1 << 23) + 1) is None
    out = (ctypes.c_int32 * 4)()
    assert L.pkv_pool_admit(None, None, 0, out, 1, out, out) == pk.PKV_ERR_NULL
    assert L.pkv_pool_alloc(None, 1, out) == pk.PKV_ERR_NULL
    assert L.pkv_pool_release(None, out, 1) == pk.PKV_ERR_NULL
    assert L.pkv_pool_defrag(None, 0, out, out, out, out) == pk.PKV_ERR_NULL
    pool = pk.pkv_pool_create(4)
    try:
        assert L.pkv_pool_alloc(pool, -1, out) == pk.PKV_ERR_SHAPE
        assert L.pkv_pool_release(pool, out, -1) == pk.PKV_ERR_SHAPE
        assert pk.pkv_status_string(pk.PKV_ERR_SPACE) and pk.pkv_status_string(pk.PKV_ERR_STATE)
    finally:
        pk.pkv_pool_destroy(pool)


def test_page_hint_sizes_the_workspace_for_more_splits(pk):
    """A batch referencing fewer pages than B x W is cut into shorter splits:
    more partial slots, so at least as much workspace; no hint plans as if
    every row were full."""
    full = pk.pkv_attn_workspace_bytes(good_shape(pk, num_seqs=16, total_q=16, max_pages_per_seq=64))
    same = pk.pkv_attn_workspace_bytes(good_shape(pk, num_seqs=16, total_q=16, max_pages_per_seq=64,
                                                  total_pages=16 * 64))
    ragged = pk.pkv_attn_workspace_bytes(good_shape(pk, num_seqs=16, total_q=16, max_pages_per_seq=64,
                                                    total_pages=200))
    assert full == same > 0
    assert ragged > full


def test_host_plan_counts_pages_and_picks_a_split_length(pk):
    """pkv_attn_plan: total_pages = sum of ceil(seq_len / 256) (lengths past the
    table clipped to it, negative ones as 0); a uniform batch of full rows
    keeps the split length that fills one round exactly (8 x 32 pages, 8 KV
    heads: 8 pages, 256 workgroups); the choice stays within 1..min(W, 64)."""
    s = good_shape(pk, num_seqs=8, max_pages_per_seq=32, total_q=48, max_q_len=6)
    pk.pkv_attn_plan(s, [8192] * 8)
    assert (s.total_pages, s.pages_per_split) == (256, 8)
    s = good_shape(pk, num_seqs=5, max_pages_per_seq=64, total_q=5)
    pk.pkv_attn_plan(s, [1, 257, 16384, 99999, -3])
    assert s.total_pages == 1 + 2 + 64 + 64 + 0
    assert 1 <= s.pages_per_split <= 64
    assert pk.pkv_attn_workspace_bytes(s) > 0
    prefill = good_shape(pk, num_seqs=1, max_pages_per_seq=8, total_q=300, max_q_len=300)
    pk.pkv_attn_plan(prefill, [600])
    assert (prefill.total_pages, prefill.pages_per_split) == (3, 0)
    # a batch far too small to fill the chip keeps whole sequences (a split
    # would add a merge and shorten nothing): configuration 1's shape
    tiny = good_shape(pk, num_seqs=1, num_q_heads=8, num_kv_heads=2, head_dim=64, num_pages=16,
                      max_pages_per_seq=2, total_q=1)
    pk.pkv_attn_plan(tiny, [300])
    assert (tiny.total_pages, tiny.pages_per_split) == (2, 2)
    # and the batched-decode mix (64 sequences of 2-4 pages, 8 KV heads) one
    # split per sequence: 512 workgroups, two per CU
    mix = good_shape(pk, num_seqs=64, max_pages_per_seq=4, num_pages=256, total_q=64)
    pk.pkv_attn_plan(mix, [512 + (37 * i) % 513 for i in range(64)])
    assert mix.pages_per_split == 4


def test_host_plan_rejects_bad_input(pk):
    s = good_shape(pk)
    assert pk.LIB.pkv_attn_plan(None, None) == pk.PKV_ERR_NULL
    assert pk.LIB.pkv_attn_plan(ctypes.byref(s), None) == pk.PKV_ERR_NULL
    bad = good_shape(pk, head_dim=96)
    lens = (ctypes.c_int32 * 4)(1, 2, 3, 4)
    assert pk.LIB.pkv_attn_plan(ctypes.byref(bad), lens) == pk.PKV_ERR_SHAPE
    with pytest.raises(ValueError):
        pk.pkv_attn_plan(s, [1, 2])


def test_binding_refuses_tensors_of_another_size(pk):
    """The kernels index every buffer by the shape, so the binding checks each
    tensor's element count against it before anything reaches the device
    (CPU tensors suffice: the count is checked first)."""
    import torch
    bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    s = good_shape(pk, num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=64, num_pages=4, max_pages_per_seq=3,
                   total_q=3, max_q_len=2)
    args = dict(q=torch.zeros(3, 8, 64, dtype=bf), k_pool=torch.zeros(4, 2, 256, 64, dtype=bf),
                v_pool=torch.zeros(4, 2, 256, 64, dtype=bf), block_table=torch.zeros(2, 3, dtype=i32),
                seq_lens=torch.zeros(2, dtype=i32), q_lens=torch.zeros(2, dtype=i32),
                out=torch.zeros(3, 8, 64, dtype=f32))
    for name, bad in (("q", torch.zeros(2, 8, 64, dtype=bf)), ("out", torch.zeros(3, 8, 32, dtype=f32)),
                      ("v_pool", torch.zeros(3, 2, 256, 64, dtype=bf)), ("block_table", torch.zeros(2, 2, dtype=i32)),
                      ("q_lens", torch.zeros(3, dtype=i32))):
        a = dict(args, **{name: bad})
        with pytest.raises(ValueError, match=name):
            pk.pkv_attn_fwd(a["q"], a["k_pool"], a["v_pool"], a["block_table"], a["seq_lens"], a["q_lens"],
                            a["out"], s, torch.zeros(16, dtype=torch.uint8))
        with pytest.raises(ValueError, match=name):
            pk.pkv_attn_fwd_shared(a["q"], a["k_pool"], a["v_pool"], a["block_table"], a["seq_lens"],
                                   a["q_lens"], a["out"], s, 1, torch.zeros(16, dtype=torch.uint8))
    acc = pk.pkv_accept_shape(2, 100, 5, 4)
    with pytest.raises(ValueError, match="logits"):
        pk.pkv_accept(torch.zeros(4, 100), torch.zeros(3, dtype=i32), torch.zeros(2, dtype=i32),
                      torch.zeros(2, dtype=i32), torch.zeros(2, dtype=i32), None, acc, torch.zeros(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="draft_ids"):
        pk.pkv_accept(torch.zeros(5, 100), torch.zeros(2, dtype=i32), torch.zeros(2, dtype=i32),
                      torch.zeros(2, dtype=i32), torch.zeros(2, dtype=i32), None, acc, torch.zeros(8, dtype=torch.uint8))
    kv = pk.pkv_kv_shape(2, 2, 64, 256, 4, 3, 3)
    with pytest.raises(ValueError, match="free_pages"):
        pk.pkv_kv_append(torch.zeros(3, 2, 64, dtype=bf), torch.zeros(3, 2, 64, dtype=bf), args["k_pool"],
                         args["v_pool"], args["block_table"], args["seq_lens"], args["q_lens"],
                         torch.zeros(3, dtype=i32), torch.zeros(1, dtype=i32), kv, torch.zeros(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="accepted"):
        pk.pkv_kv_rollback(args["block_table"], args["seq_lens"], args["q_lens"], torch.zeros(1, dtype=i32),
                           torch.zeros(4, dtype=i32), torch.zeros(1, dtype=i32), kv, torch.zeros(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="dst"):
        pk.pkv_pool_copy_pages(args["k_pool"], args["v_pool"], torch.zeros(2, dtype=i32), torch.zeros(3, dtype=i32))


def _shared_prefix_reference(table, seq_lens, q_lens):
    """The shared-prefix contract written out: the largest n < W with every
    row's first n entries equal to row 0's and seq_len - q_len >= 256 n on
    every row with a window; 0 without any window."""
    B, W = table.shape
    if not (q_lens > 0).any():
        return 0
    best = 0
    for n in range(W):
        ok = all((table[b, :n] == table[0, :n]).all() for b in range(B))
        ok = ok and all(seq_lens[b] - q_lens[b] >= 256 * n for b in range(B) if q_lens[b] > 0)
        if ok:
            best = n
    return best


def test_shared_prefix_pages_from_host_tables(pk):
    rng = np.random.default_rng(5)
    for trial in range(200):
        B, W = int(rng.integers(1, 6)), int(rng.integers(1, 7))
        base = rng.integers(0, 50, W)
        table = np.tile(base, (B, 1)).astype(np.int32)
        for b in range(B):                       # each row diverges somewhere, or not at all
            cut = int(rng.integers(0, W + 1))
            table[b, cut:] = rng.integers(50, 100, W - cut)
        q_lens = rng.integers(0, 4, B).astype(np.int32)
        seq_lens = (q_lens + rng.integers(0, W * 256 - 3, B)).astype(np.int32)
        s = good_shape(pk, num_seqs=B, max_pages_per_seq=W, total_q=int(q_lens.sum()), max_q_len=4)
        assert pk.pkv_shared_prefix_pages(table, seq_lens, q_lens, s) == \
            _shared_prefix_reference(table, seq_lens, q_lens), trial
    with pytest.raises(ValueError):
        pk.pkv_shared_prefix_pages(np.zeros((2, 3), np.int32), [1], [1], good_shape(pk, num_seqs=2,
                                                                                      max_pages_per_seq=3))
    assert pk.LIB.pkv_shared_prefix_pages(None, None, None, None) == pk.PKV_ERR_NULL


def test_quantized_calls_check_shapes_pointers_and_workspace(pk):
    """The Q8 / Q4 entry points refuse bad input before any launch: unsupported
    head sizes and row counts in the encoders, long windows, missing scale
    pools and short workspaces in attention, and the cache appends' pointer
    and workspace checks."""
    d = ctypes.c_void_p(0x1000)
    for enc in (pk.LIB.pkv_q8_encode, pk.LIB.pkv_q4_encode):
        assert enc(d, d, d, 10, 96, None) == pk.PKV_ERR_SHAPE
        assert enc(d, d, d, -1, 128, None) == pk.PKV_ERR_SHAPE
        assert enc(d, d, d, (1 << 32) + 1, 128, None) == pk.PKV_ERR_SHAPE
        assert enc(None, d, d, 10, 128, None) == pk.PKV_ERR_NULL
        assert enc(None, None, None, 0, 64, None) == pk.PKV_OK
    s = good_shape(pk)
    need = pk.pkv_attn_workspace_bytes(s)
    for fwd in (pk.LIB.pkv_attn_fwd_q8, pk.LIB.pkv_attn_fwd_q4):
        assert fwd(*([d] * 9), None, d, need, None) == pk.PKV_ERR_NULL
        assert fwd(d, d, None, d, d, d, d, d, d, ctypes.byref(s), d, need, None) == pk.PKV_ERR_NULL  # k scales
        assert fwd(*([d] * 9), ctypes.byref(s), d, need - 1, None) == pk.PKV_ERR_WORKSPACE
        long = good_shape(pk)
        long.max_q_len = 64          # 64 window rows x the group: past the decode / verify tile
        assert fwd(*([d] * 9), ctypes.byref(long), d, 1 << 30, None) == pk.PKV_ERR_SHAPE
        empty = good_shape(pk, num_seqs=0, total_q=0)
        assert fwd(*([None] * 9), ctypes.byref(empty), None, 0, None) == pk.PKV_OK
    ks = pk.pkv_kv_shape(4, 8, 128, 256, 256, 32, 24)
    kneed = pk.pkv_kv_workspace_bytes(ks)
    for app in (pk.LIB.pkv_kv_append_q8, pk.LIB.pkv_kv_append_q4):
        assert app(*([d] * 11), ctypes.byref(ks), d, kneed - 1, None) == pk.PKV_ERR_WORKSPACE
        assert app(d, d, d, None, d, d, d, d, d, d, d, ctypes.byref(ks), d, kneed, None) == pk.PKV_ERR_NULL
        assert app(*([d] * 11), None, d, kneed, None) == pk.PKV_ERR_NULL
        empty = pk.pkv_kv_shape(0, 8, 128, 256, 256, 32, 0)
        assert app(*([None] * 11), ctypes.byref(empty), None, 0, None) == pk.PKV_OK


def test_byte_page_moves_check_sizes_and_pointers(pk):
    d = ctypes.c_void_p(0x1000)
    f = pk.LIB.pkv_pool_copy_page_bytes
    assert f(d, d, d, d, 1, 16, 24, None, None) == pk.PKV_ERR_SHAPE         # not a multiple of 16
    assert f(d, d, d, d, 1, 16, 0, None, None) == pk.PKV_ERR_SHAPE
    assert f(d, d, d, d, -1, 16, 4096, None, None) == pk.PKV_ERR_SHAPE
    assert f(d, d, d, d, 1, 1 << 20, 1 << 21, None, None) == pk.PKV_ERR_SHAPE   # 2^41 bytes of pool
    assert f(d, None, d, d, 1, 16, 4096, None, None) == pk.PKV_ERR_NULL
    assert f(None, None, None, None, 0, 16, 4096, None, None) == pk.PKV_OK


def test_accept_noalloc_refuses_shapes_past_its_scratch_before_any_launch(pk):
    # host-side check only: the pointers are never dereferenced
    shape = pk.pkv_accept_shape(4000, 1 << 20, 4000, 0)
    assert pk.pkv_accept_workspace_bytes(shape) > pk.PKV_ACCEPT_SCRATCH_BYTES
    fake = ctypes.c_void_p(256)
    rc = pk.LIB.pkv_accept_noalloc(fake, fake, fake, fake, fake, None, ctypes.byref(shape), None)
    assert rc == pk.PKV_ERR_SCRATCH
    assert "scratch" in pk.pkv_status_string(rc)
    assert pk.LIB.pkv_accept_noalloc(fake, fake, fake, fake, fake, None, None, None) == pk.PKV_ERR_NULL
