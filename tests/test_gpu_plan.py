"""Ragged batches and the split plan (pkv_attn_shape.total_pages and
pages_per_split, pkv_attn_plan): the plan only decides how the key range is
cut into splits, so every hint (none, exact, far too small, far too large),
every forced split length and the host plan's own choice must give the
oracle's result on a batch whose lengths span 2 to 16384 tokens in a
64-page-wide table; and the mixed job queue's first steps with the host plan."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
from workloads import normal_bf16, AttnCase, BF16_QNAN, Config5Queue
from tests.gpu_util import say, attn_gpu, assert_close


@pytest.fixture(scope="module")
def pk():
    import torch
    assert torch.cuda.is_available()
    import paged_kv_attention_attn_amd as pk
    return pk


def pages_of(seq_lens):
    return int(sum(-(-int(n) // 256) for n in seq_lens))


def ragged_case(seed, lens, q_lens, Hq=32, Hkv=8, D=128, W=64):
    rng = np.random.default_rng(seed)
    own = [-(-n // 256) for n in lens]
    P = sum(own) + 5
    perm = rng.permutation(P).astype(np.int32)
    table = np.full((len(lens), W), -1, np.int32)
    o = 0
    for b, n in enumerate(own):
        table[b, :n] = perm[o:o + n]
        o += n
    k = normal_bf16(rng, (P, Hkv, 256, D))
    v = normal_bf16(rng, (P, Hkv, 256, D))
    for p in perm[o:]:
        k[p] = BF16_QNAN
        v[p] = BF16_QNAN
    for b, n in enumerate(lens):
        fill = n % 256
        if fill:
            last = int(table[b, own[b] - 1])
            k[last, :, fill:] = BF16_QNAN
            v[last, :, fill:] = BF16_QNAN
    q_lens = np.asarray(q_lens, np.int32)
    q = normal_bf16(rng, (int(q_lens.sum()), Hq, D))
    return AttnCase("ragged", q, k, v, table, np.asarray(lens, np.int32), q_lens,
                    float(np.float32(1 / np.sqrt(D))))


LENS = [16384, 300, 1000, 256, 5000, 2, 700, 9000, 4097, 60]
QLENS = [7, 1, 3, 5, 1, 1, 7, 3, 5, 1]


@pytest.fixture(scope="module")
def ragged():
    case = ragged_case(31, LENS, QLENS)
    ref = oracle.attention(case.q, case.k_pool, case.v_pool, case.block_table, case.seq_lens, case.q_lens,
                           case.scale)
    return case, ref


@pytest.mark.parametrize("hint", ["none", "exact", "one", "tenfold"])
def test_every_page_hint_gives_the_oracle_result(pk, ragged, hint):
    case, ref = ragged
    exact = pages_of(case.seq_lens)
    total = {"none": 0, "exact": exact, "one": 1, "tenfold": 10 * exact}[hint]
    say(f"ragged batch, {len(LENS)} sequences, {exact} pages, hint {hint} ({total})")
    got, flags = attn_gpu(case, pk, total_pages=total)
    assert flags == 0
    assert_close(got, ref, f"ragged hint {hint}")


@pytest.mark.parametrize("pps", [1, 3, 64])
def test_forced_split_lengths_give_the_oracle_result(pk, ragged, pps):
    case, ref = ragged
    say(f"ragged batch, pages_per_split {pps}")
    got, flags = attn_gpu(case, pk, pages_per_split=pps)
    assert flags == 0
    assert_close(got, ref, f"ragged pps {pps}")


def test_host_plan_gives_the_oracle_result(pk, ragged):
    case, ref = ragged
    say("ragged batch, host plan")
    got, flags = attn_gpu(case, pk, plan=True)
    assert flags == 0
    assert_close(got, ref, "ragged host plan")


def test_job_queue_steps_with_the_host_plan(pk):
    q = Config5Queue(seed=0)
    ref = {}
    for st in q.steps():
        if st.index >= 3:
            break
        c = st.case
        say(f"job queue step {st.index} with the host plan: {c.num_seqs} sequences")
        got, flags = attn_gpu(c, pk, plan=True)
        assert flags == 0
        r0 = 0
        for b, jid in enumerate(st.job_ids):
            ql = int(c.q_lens[b])
            if jid not in ref:
                jc, _ = q.job_case(jid)
                ref[jid] = oracle.attention(jc.q, jc.k_pool, jc.v_pool, jc.block_table, jc.seq_lens, jc.q_lens,
                                            jc.scale)
            assert_close(got[r0:r0 + ql], ref[jid], f"queue step {st.index} job {jid}")
            r0 += ql
