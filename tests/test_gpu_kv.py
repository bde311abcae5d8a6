"""GPU parity of the cache append and rollback calls with the oracle
(bit-exact: pools, tables, lengths and the free stack), their all-or-nothing
contract checks, and a multi-step speculative verify loop (append ->
attention -> accept -> rollback) against the oracle doing the same steps."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
from oracle import kv_cache as kv
from workloads import normal_bf16, make_accept_case
from tests.gpu_util import say, dev_bf16, dev_i32, assert_close
from tests.test_oracle_kv import random_state


@pytest.fixture(scope="module")
def pk():
    import torch
    assert torch.cuda.is_available()
    import paged_kv_attention_attn_amd as pk
    return pk


class DevCache:
    """Cache state on the GPU: pools, tables, lengths and the free stack."""

    def __init__(self, pk, kp, vp, table, lens, free, count, total_q):
        import torch
        self.pk, self.torch = pk, torch
        self.k, self.v = dev_bf16(kp), dev_bf16(vp)
        self.table, self.lens, self.free = dev_i32(table), dev_i32(lens), dev_i32(free)
        self.count = dev_i32(np.array([count]))
        self.shape = pk.kv_shape(self.k, self.table, total_q)
        self.ws = pk.new_kv_workspace(self.shape)

    def append(self, kn, vn, ql):
        self.pk.pkv_kv_append(dev_bf16(kn), dev_bf16(vn), self.k, self.v, self.table, self.lens, dev_i32(ql),
                              self.free, self.count, self.shape, self.ws)

    def rollback(self, ql, acc):
        acc_t = acc if hasattr(acc, "data_ptr") else dev_i32(acc)
        self.pk.pkv_kv_rollback(self.table, self.lens, dev_i32(ql), acc_t, self.free, self.count, self.shape,
                                self.ws)

    def host(self):
        self.torch.cuda.synchronize()
        bits = lambda t: t.view(self.torch.int16).cpu().numpy().view(np.uint16)
        c = int(self.count.cpu()[0])
        return bits(self.k), bits(self.v), self.table.cpu().numpy(), self.lens.cpu().numpy(), \
            self.free.cpu().numpy(), c

    def errors(self):
        return self.pk.pkv_kv_check_errors(self.ws)


def check_equal(dc, k, v, table, lens, free, count, what):
    gk, gv, gt, gl, gf, gc = dc.host()
    np.testing.assert_array_equal(gt, table, err_msg=f"{what}: table")
    np.testing.assert_array_equal(gl, lens, err_msg=f"{what}: lengths")
    assert gc == count, f"{what}: free count {gc} != {count}"
    np.testing.assert_array_equal(gf[:gc], free[:count], err_msg=f"{what}: free stack")
    assert np.array_equal(gk, k), f"{what}: K pool differs"
    assert np.array_equal(gv, v), f"{what}: V pool differs"


@pytest.mark.parametrize("seed,D", [(0, 128), (1, 128), (2, 64), (3, 128)])
def test_append_and_rollback_match_the_oracle(pk, seed, D):
    say(f"kv append/rollback parity seed {seed} D {D}")
    kp, vp, table, lens, ql, kn, vn, free, cnt = random_state(seed, B=6, P=48, W=8, Hkv=8, D=D, max_q=16)
    dc = DevCache(pk, kp, vp, table, lens, free, cnt, int(ql.sum()))
    dc.append(kn, vn, ql)
    k2, v2, t2, l2, f2, c2 = kv.append(kp, vp, table, lens, ql, kn, vn, free, cnt)
    check_equal(dc, k2, v2, t2, l2, f2, c2, "append")
    acc = np.array([np.random.default_rng(seed).integers(0, q + 1) for q in ql], np.int32)
    dc.rollback(ql, acc)
    t3, l3, f3, c3 = kv.rollback(t2, l2, ql, acc, f2, c2)
    check_equal(dc, k2, v2, t3, l3, f3, c3, "rollback")
    assert dc.errors() == 0


def test_many_sequences_and_an_empty_window(pk):
    say("kv: 1500 sequences (two plan tiles), some windows empty")
    rng = np.random.default_rng(9)
    B, P, W, Hkv, D = 1500, 4096, 4, 2, 64
    lens = rng.integers(0, 3 * 256, B).astype(np.int32)
    ql = rng.integers(0, 8, B).astype(np.int32)
    perm = rng.permutation(P).astype(np.int32)
    table = np.full((B, W), -1, np.int32)
    used = 0
    for b in range(B):
        n = -(-int(lens[b]) // 256)
        table[b, :n] = perm[used:used + n]
        used += n
    free = np.full(P, -1, np.int32)
    free[:P - used] = perm[used:]
    kp = rng.integers(0, 2**16, (P, Hkv, 256, D), dtype=np.uint16)
    vp = kp ^ np.uint16(0x5555)
    kn = rng.integers(0, 2**16, (int(ql.sum()), Hkv, D), dtype=np.uint16)
    vn = kn ^ np.uint16(0x3333)
    dc = DevCache(pk, kp, vp, table, lens, free, P - used, int(ql.sum()))
    dc.append(kn, vn, ql)
    k2, v2, t2, l2, f2, c2 = kv.append(kp, vp, table, lens, ql, kn, vn, free, P - used)
    check_equal(dc, k2, v2, t2, l2, f2, c2, "append")
    acc = (ql // 2).astype(np.int32)
    dc.rollback(ql, acc)
    t3, l3, f3, c3 = kv.rollback(t2, l2, ql, acc, f2, c2)
    check_equal(dc, k2, v2, t3, l3, f3, c3, "rollback")


def test_broken_contracts_change_nothing(pk):
    say("kv: broken contracts set flags and change nothing")
    kp, vp, table, lens, ql, kn, vn, free, cnt = random_state(5, B=4, P=24, W=6, Hkv=2, D=64, max_q=7)
    ql[0] = 3
    rows = int(ql.sum())
    rng = np.random.default_rng(5)
    kn = rng.integers(0, 2**16, (rows + 1, 2, 64), dtype=np.uint16)
    vn = rng.integers(0, 2**16, (rows + 1, 2, 64), dtype=np.uint16)
    base = (kp, vp, table, lens, free)

    dc = DevCache(pk, kp, vp, table, lens, free, 0, rows)       # no free page at all
    need = sum(-(-int(l + q) // 256) - (-(-int(l) // 256)) for l, q in zip(lens, ql))
    dc.append(kn[:rows], vn[:rows], ql)
    if need:
        check_equal(dc, *base, 0, "no free pages")
        assert dc.errors() & pk.PKV_EFLAG_SPACE

    dc = DevCache(pk, kp, vp, table, lens, free, cnt, rows + 1)  # rows do not add up
    dc.append(kn, vn, ql)
    check_equal(dc, *base, cnt, "row count")
    assert dc.errors() & pk.PKV_EFLAG_ROWS

    bad = lens.copy()
    bad[0] = table.shape[1] * 256 - 1                              # window runs past the table row
    dc = DevCache(pk, kp, vp, table, bad, free, cnt, rows)
    dc.append(kn[:rows], vn[:rows], ql)
    check_equal(dc, kp, vp, table, bad, free, cnt, "table overflow")
    assert dc.errors() & pk.PKV_EFLAG_QLEN

    dc = DevCache(pk, kp, vp, table, lens + ql, free, cnt, rows)
    dc.rollback(ql, ql + 1)                                        # more accepted than drafted
    check_equal(dc, kp, vp, table, lens + ql, free, cnt, "rollback")
    assert dc.errors() & pk.PKV_EFLAG_QLEN


def test_speculative_verify_loop(pk):
    """Five verify steps on four sequences: append the window's K/V, attend,
    accept against planted drafts, roll back to the accepted prefix. The
    oracle runs the same steps on the CPU; every step must agree."""
    import torch
    say("kv: speculative verify loop, 5 steps")
    rng = np.random.default_rng(77)
    B, Hq, Hkv, D, P, W, V = 4, 8, 2, 128, 64, 12, 4000
    lens = np.array([255, 256, 700, 1], np.int32)
    perm = rng.permutation(P).astype(np.int32)
    table = np.full((B, W), -1, np.int32)
    used = 0
    for b in range(B):
        n = -(-int(lens[b]) // 256)
        table[b, :n] = perm[used:used + n]
        used += n
    free = np.full(P, -1, np.int32)
    free[:P - used] = perm[used:]
    kp = normal_bf16(rng, (P, Hkv, 256, D))
    vp = normal_bf16(rng, (P, Hkv, 256, D))
    state = (kp, vp, table, lens, free, P - used)
    dc = DevCache(pk, kp, vp, table, lens, free, P - used, 0)
    window = np.full(B, 5, np.int32)
    scale = 1.0 / np.sqrt(D)
    for step in range(5):
        ql = np.minimum(window, 15).astype(np.int32) + 1            # n drafts + the last token
        ql[step % B] = 1                                             # a plain decode row now and then
        rows = int(ql.sum())
        kn, vn = normal_bf16(rng, (rows, Hkv, D)), normal_bf16(rng, (rows, Hkv, D))
        q = normal_bf16(rng, (rows, Hq, D))
        acc_case = make_accept_case(100 + step, ql, V)
        # oracle
        kp, vp, table, lens, free, cnt = state
        k2, v2, t2, l2, f2, c2 = kv.append(kp, vp, table, lens, ql, kn, vn, free, cnt)
        ref_out = oracle.attention(q, k2, v2, t2, l2, ql, scale)
        ea, en, _ = oracle.accept(acc_case.logits, acc_case.draft_ids, acc_case.n_draft)
        t3, l3, f3, c3 = kv.rollback(t2, l2, ql, ea, f2, c2)
        state = (k2, v2, t3, l3, f3, c3)
        # GPU
        dc.shape = pk.kv_shape(dc.k, dc.table, rows)
        dc.ws = pk.new_kv_workspace(dc.shape)
        dc.append(kn, vn, ql)
        qd = dev_bf16(q)
        out = torch.empty((rows, Hq, D), dtype=torch.float32, device="cuda")
        ashape = pk.attn_shape(qd, dc.k, dc.table, int(ql.max()), scale)
        aws = pk.new_attn_workspace(ashape)
        pk.pkv_attn_fwd(qd, dc.k, dc.v, dc.table, dc.lens, dev_i32(ql), out, ashape, aws)
        logits = torch.from_numpy(np.ascontiguousarray(acc_case.logits)).cuda()
        nd = dev_i32(acc_case.n_draft)
        oa = torch.empty(B, dtype=torch.int32, device="cuda")
        on = torch.empty_like(oa)
        cshape = pk.accept_shape(logits, nd, int(acc_case.n_draft.max()))
        pk.pkv_accept(logits, dev_i32(acc_case.draft_ids), nd, oa, on, None, cshape,
                      pk.new_accept_workspace(cshape))
        dc.rollback(ql, oa)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref_out, f"verify step {step}")
        np.testing.assert_array_equal(oa.cpu().numpy(), ea)
        np.testing.assert_array_equal(on.cpu().numpy(), en)
        check_equal(dc, k2, v2, t3, l3, f3, c3, f"verify step {step}")
        assert dc.errors() == 0 and pk.pkv_attn_check_errors(aws) == 0
        window = oracle.window_next(window, ql - 1, ea).astype(np.int32)
