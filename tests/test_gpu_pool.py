"""GPU side of the page allocator: page copies and block-table remaps against
the oracle (bit-exact), their contract checks, and a whole defragmentation:
jobs admitted by the library's allocator over a shared prefix, attention
before and after moving every occupied page down and rewriting the tables
must agree bit for bit."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
from oracle import page_pool as opool
from workloads import normal_bf16
from tests.gpu_util import say, dev_bf16, dev_i32


@pytest.fixture(scope="module")
def pk():
    import torch
    assert torch.cuda.is_available()
    import paged_kv_attention_attn_amd as pk
    return pk


def bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("Hkv,D", [(8, 128), (2, 64), (3, 64)])
def test_copy_pages_matches_the_oracle(pk, Hkv, D):
    import torch
    say(f"pool copy pages Hkv={Hkv} D={D}")
    rng = np.random.default_rng(Hkv * 1000 + D)
    P = 40
    k = rng.integers(0, 2**16, (P, Hkv, 256, D), dtype=np.uint16)
    v = rng.integers(0, 2**16, (P, Hkv, 256, D), dtype=np.uint16)
    perm = rng.permutation(P)
    moves = list(zip(perm[20:33].tolist(), perm[:13].tolist()))     # 13 disjoint moves
    kd, vd = dev_bf16(k), dev_bf16(v)
    src = dev_i32([s for s, _ in moves])
    dst = dev_i32([d for _, d in moves])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pk.pkv_pool_copy_pages(kd, vd, src, dst, err)
    torch.cuda.synchronize()
    k2, v2 = opool.copy_pages(k, v, moves)
    assert np.array_equal(bits(kd), k2) and np.array_equal(bits(vd), v2)
    assert int(err.item()) == 0


def test_copy_pages_skips_bad_entries(pk):
    import torch
    say("pool copy pages: an entry outside the pool")
    rng = np.random.default_rng(3)
    k = rng.integers(0, 2**16, (6, 2, 256, 64), dtype=np.uint16)
    kd, vd = dev_bf16(k), dev_bf16(k ^ np.uint16(0x1111))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pk.pkv_pool_copy_pages(kd, vd, dev_i32([5, 9]), dev_i32([0, 1]), err)
    torch.cuda.synchronize()
    k2, _ = opool.copy_pages(k, k, [(5, 0)])
    assert np.array_equal(bits(kd), k2)
    assert int(err.item()) & pk.PKV_EFLAG_PAGE


def test_table_remap_matches_the_oracle(pk):
    import torch
    say("pool table remap")
    rng = np.random.default_rng(4)
    P = 300
    table = rng.integers(-1, P, (37, 19)).astype(np.int32)
    remap = rng.permutation(P).astype(np.int32)
    td = dev_i32(table)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pk.pkv_table_remap(td, dev_i32(remap), err)
    torch.cuda.synchronize()
    assert np.array_equal(td.cpu().numpy(), opool.remap_table(table, remap.tolist()))
    assert int(err.item()) == 0
    bad = table.copy()
    bad[3, 4] = P + 2
    td = dev_i32(bad)
    pk.pkv_table_remap(td, dev_i32(remap), err)
    torch.cuda.synchronize()
    got = td.cpu().numpy()
    assert got[3, 4] == P + 2 and int(err.item()) & pk.PKV_EFLAG_PAGE
    want = opool.remap_table(np.where(bad >= P, -1, bad), remap.tolist())
    mask = bad < P
    assert np.array_equal(got[mask], want[mask])


def test_defragmentation_keeps_attention_bit_exact(pk):
    """Jobs with a shared 600-token prefix and private tails are admitted by
    the library allocator into a churned 64-page pool; after a full
    defragmentation (every occupied page moved below the occupied count, the
    contents copied and the tables remapped on the GPU), attention over every
    job gives the same bits as before."""
    import torch
    say("pool: defragmentation end to end")
    rng = np.random.default_rng(11)
    P, Hq, Hkv, D = 64, 8, 2, 128
    pool = pk.pkv_pool_create(P)
    prefix = rng.integers(0, 32000, 600).tolist()
    jobs = []
    for i in range(14):
        pages, cached = pk.pkv_pool_admit(pool, prefix + rng.integers(0, 32000, int(rng.integers(1, 700))).tolist())
        jobs.append(pages)
        if i % 3 == 2:                       # churn: finish an earlier job
            pk.pkv_pool_release(pool, jobs.pop(0))
    for j in (5, 2):                         # finished jobs in the middle leave holes
        pk.pkv_pool_release(pool, jobs.pop(j))
    k = normal_bf16(rng, (P, Hkv, 256, D))
    v = normal_bf16(rng, (P, Hkv, 256, D))
    W = max(len(j) for j in jobs)
    table = np.full((len(jobs), W), -1, np.int32)
    lens = np.zeros(len(jobs), np.int32)
    for b, pages in enumerate(jobs):
        table[b, :len(pages)] = pages
        lens[b] = 256 * (len(pages) - 1) + int(rng.integers(1, 257))
    q_lens = np.full(len(jobs), 3, np.int32)
    q = normal_bf16(rng, (int(q_lens.sum()), Hq, D))
    kd, vd, td, qd = dev_bf16(k), dev_bf16(v), dev_i32(table), dev_bf16(q)
    sl, ql = dev_i32(lens), dev_i32(q_lens)
    shape = pk.attn_shape(qd, kd, td, 3, 1.0 / np.sqrt(D))
    ws = pk.new_attn_workspace(shape)
    out0 = torch.empty((int(q_lens.sum()), Hq, D), dtype=torch.float32, device="cuda")
    pk.pkv_attn_fwd(qd, kd, vd, td, sl, ql, out0, shape, ws)
    remap, moves = pk.pkv_pool_defrag(pool, P, move_referenced=True)
    assert moves, "the churn should leave holes below the occupied count"
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pk.pkv_pool_copy_pages(kd, vd, dev_i32([s for s, _ in moves]), dev_i32([d for _, d in moves]), err)
    pk.pkv_table_remap(td, dev_i32(remap), err)
    out1 = torch.empty_like(out0)
    pk.pkv_attn_fwd(qd, kd, vd, td, sl, ql, out1, shape, ws)
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and pk.pkv_attn_check_errors(ws) == 0
    assert torch.equal(out0, out1)
    n_occ = P - pk.pkv_pool_stats(pool)[0]
    t = td.cpu().numpy()
    assert t[t >= 0].max() < n_occ
    assert np.array_equal(t, opool.remap_table(table, remap))
    ref = oracle.attention(q, k, v, table, lens, q_lens, 1.0 / np.sqrt(D))
    assert np.allclose(out1.cpu().numpy(), ref, atol=2e-3, rtol=1e-2)
    pk.pkv_pool_destroy(pool)
