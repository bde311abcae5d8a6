"""The allocation-free accept entry point (pkv_accept_noalloc) against
pkv_accept on the same inputs: argmax, accepted count, next token and window
bit-exact, on two calls in a row (the second with fewer rows and a smaller
vocabulary), then once more at the larger shape, so a call that left its
fixed scratch dirty would show."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

from workloads import make_config, make_accept_case
from tests.gpu_util import say


@pytest.fixture(scope="module")
def pk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_attention_attn_amd as pk
    return pk


def run_both(pk, acc):
    import torch
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    logits = torch.from_numpy(np.ascontiguousarray(acc.logits, dtype=np.float32)).cuda()
    drafts, nd = i32(acc.draft_ids), i32(acc.n_draft)
    shape = pk.accept_shape(logits, nd, acc.max_draft)
    assert pk.pkv_accept_workspace_bytes(shape) <= pk.PKV_ACCEPT_SCRATCH_BYTES
    out = {}
    for name in ("workspace", "noalloc"):
        oa = torch.full((acc.num_seqs,), -7, dtype=torch.int32, device="cuda")
        on = torch.full_like(oa, -7)
        win = i32(acc.window)
        if name == "workspace":
            pk.pkv_accept(logits, drafts, nd, oa, on, win, shape, pk.new_accept_workspace(shape))
        else:
            pk.pkv_accept_noalloc(logits, drafts, nd, oa, on, win, shape)
        torch.cuda.synchronize()
        out[name] = (oa.cpu().numpy(), on.cpu().numpy(), win.cpu().numpy())
    for a, b in zip(out["workspace"], out["noalloc"]):
        np.testing.assert_array_equal(a, b)
    return out["noalloc"]


def test_noalloc_matches_the_workspace_call_on_consecutive_shapes(pk):
    _, big = make_config(3)                      # 8 sequences x 6 rows over 128256 logits
    small = make_accept_case(21, [3, 1, 2], 32000)
    say("accept without allocation: verify shape 48 x 128256")
    oa, _, _ = run_both(pk, big)
    np.testing.assert_array_equal(oa, big.planted_match + 1)
    say("accept without allocation: smaller shape 6 x 32000 right after")
    run_both(pk, small)
    say("accept without allocation: the large shape again")
    run_both(pk, big)


def test_noalloc_refuses_shapes_past_its_scratch(pk):
    import torch
    rows, vocab = 4000, 1 << 20
    shape = pk.pkv_accept_shape(rows, vocab, rows, 0)
    assert pk.pkv_accept_workspace_bytes(shape) > pk.PKV_ACCEPT_SCRATCH_BYTES
    dummy = torch.zeros(16, dtype=torch.int32, device="cuda")
    rc = pk.LIB.pkv_accept_noalloc(dummy.data_ptr(), None, dummy.data_ptr(), dummy.data_ptr(),
                                   dummy.data_ptr(), None, __import__("ctypes").byref(shape), None)
    assert rc == pk.PKV_ERR_SCRATCH
