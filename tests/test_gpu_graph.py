"""Both entry points under HIP graph capture: a verify step (attention over a
split-K shape whose splits merge through the workspace counters, then the
accept over its logits) is captured once and replayed several times, with
eager work and synchronisations in between. Every replay must reproduce the
eager result bit for bit, which also shows that each call leaves its
workspace clean for the next (counters back at zero, row keys cleared)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import oracle
from workloads import make_tiny_case, make_accept_case
from tests.gpu_util import say, DeviceCase, dev_i32, assert_close


@pytest.fixture(scope="module")
def pk():
    import torch
    assert torch.cuda.is_available()
    import paged_kv_attention_attn_amd as pk
    return pk


def test_verify_step_replays_bit_exact(pk):
    import torch
    say("graph: attention (split merge) + accept, 4 replays")
    # long enough that every (sequence, KV head) is cut into several splits
    case = make_tiny_case(21, [4000, 2600, 900], [6, 4, 2], Hq=8, Hkv=2, D=128, num_pages=64)
    dc = DeviceCase(case, pk)
    acc = make_accept_case(22, [6, 4, 2], 32000)
    logits = torch.from_numpy(np.ascontiguousarray(acc.logits)).cuda()
    drafts, nd = dev_i32(acc.draft_ids), dev_i32(acc.n_draft)
    B = acc.num_seqs
    oa = torch.zeros(B, dtype=torch.int32, device="cuda")
    on = torch.zeros_like(oa)
    ashape = pk.accept_shape(logits, nd, acc.max_draft)
    aws = pk.new_accept_workspace(ashape)

    def step(stream=None):
        dc.run(stream)
        pk.pkv_accept(logits, drafts, nd, oa, on, None, ashape, aws, stream)

    # eager reference (and a check against the oracle)
    step()
    torch.cuda.synchronize()
    ref_out, ref_a, ref_n = dc.out.clone(), oa.clone(), on.clone()
    assert_close(ref_out.cpu().numpy(), oracle.attention(case.q, case.k_pool, case.v_pool, case.block_table,
                                                         case.seq_lens, case.q_lens, case.scale),
                 "graph eager")
    ea, en, _ = oracle.accept(acc.logits, acc.draft_ids, acc.n_draft)
    np.testing.assert_array_equal(ref_a.cpu().numpy(), ea)
    np.testing.assert_array_equal(ref_n.cpu().numpy(), en)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(s)  # warm the capture stream once, outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        dc.out.fill_(float("nan"))
        oa.fill_(-7)
        on.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dc.out, ref_out), f"replay {rep}: attention differs"
        assert torch.equal(oa, ref_a) and torch.equal(on, ref_n), f"replay {rep}: accept differs"
        step()  # eager work between replays, on the same workspaces
        torch.cuda.synchronize()
        assert torch.equal(dc.out, ref_out), f"eager after replay {rep}: attention differs"
    assert dc.errors() == 0


def test_shared_prefix_and_long_window_replay_bit_exact(pk):
    """The shared-prefix call (three launches: prefix splits, tails, merge)
    and a long-window call (prefill tiles) captured together; every replay
    equals the eager result bit for bit."""
    import torch
    from tests.test_gpu_shared import shared_case
    say("graph: shared-prefix call + long window, 4 replays")
    sc = shared_case(31, 3, [40, 300, 7, 256], [1, 2, 1, 3])
    sd = DeviceCase(sc, pk)
    sws = pk.new_attn_shared_workspace(sd.shape, 3)
    long_case = make_tiny_case(32, [900, 300], [200, 64], Hq=8, Hkv=2, D=128, num_pages=16)
    ld = DeviceCase(long_case, pk)

    def step():
        pk.pkv_attn_fwd_shared(sd.q, sd.k, sd.v, sd.bt, sd.sl, sd.ql, sd.out, sd.shape, 3, sws)
        ld.run()

    step()
    torch.cuda.synchronize()
    ref_s, ref_l = sd.out.clone(), ld.out.clone()
    assert_close(ref_s.cpu().numpy(), oracle.attention(sc.q, sc.k_pool, sc.v_pool, sc.block_table, sc.seq_lens,
                                                       sc.q_lens, sc.scale), "graph shared eager")
    assert_close(ref_l.cpu().numpy(), oracle.attention(long_case.q, long_case.k_pool, long_case.v_pool,
                                                       long_case.block_table, long_case.seq_lens,
                                                       long_case.q_lens, long_case.scale), "graph long eager")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        sd.out.fill_(float("nan"))
        ld.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sd.out, ref_s), f"replay {rep}: shared-prefix call differs"
        assert torch.equal(ld.out, ref_l), f"replay {rep}: long window differs"
        step()
        torch.cuda.synchronize()
        assert torch.equal(sd.out, ref_s) and torch.equal(ld.out, ref_l), f"eager after replay {rep}"
    assert pk.pkv_attn_check_errors(sws) == 0 and ld.errors() == 0


def test_two_streams_with_separate_workspaces(pk):
    """The library keeps no state outside the workspace: two batches (a verify
    shape whose splits merge through the workspace counters, and a decode
    shape) launched alternately on two streams, ten rounds, give the same bits
    as each alone."""
    import torch
    say("two streams, separate workspaces")
    a = DeviceCase(make_tiny_case(51, [4000, 2600, 900], [6, 4, 2], Hq=8, Hkv=2, D=128, num_pages=64), pk)
    b = DeviceCase(make_tiny_case(52, [3000, 700, 5000, 64], [1, 1, 1, 1], Hq=32, Hkv=8, D=128, num_pages=64), pk)
    ref_a = torch.from_numpy(a.result()).cuda()
    ref_b = torch.from_numpy(b.result()).cuda()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs_a, outs_b = [], []
    for _ in range(10):
        with torch.cuda.stream(s1):
            a.run(s1)
            outs_a.append(a.out.clone())
        with torch.cuda.stream(s2):
            b.run(s2)
            outs_b.append(b.out.clone())
    torch.cuda.synchronize()
    assert all(torch.equal(o, ref_a) for o in outs_a), "stream 1 results differ"
    assert all(torch.equal(o, ref_b) for o in outs_b), "stream 2 results differ"
    assert a.errors() == 0 and b.errors() == 0
