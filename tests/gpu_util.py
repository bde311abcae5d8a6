"""GPU-side helpers for the parity tests: upload a generated case, run the
library through its C ABI, and compare with the oracle."""

import sys

import numpy as np
import torch

TOL_ATOL = 2e-3
TOL_RTOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


class DeviceCase:
    """A case resident on the GPU plus its workspace."""

    def __init__(self, case, pk, max_q_len=None, table_width=None, total_pages=0, pages_per_split=0,
                 plan=False):
        self.case = case
        self.pk = pk
        bt = case.block_table
        if table_width is not None and table_width > bt.shape[1]:
            pad = np.full((bt.shape[0], table_width - bt.shape[1]), -1, np.int32)
            bt = np.concatenate([bt, pad], axis=1)
        self.q = dev_bf16(case.q)
        self.k = dev_bf16(case.k_pool)
        self.v = dev_bf16(case.v_pool)
        self.bt = dev_i32(bt)
        self.sl = dev_i32(case.seq_lens)
        self.ql = dev_i32(case.q_lens)
        mq = max_q_len if max_q_len is not None else max(1, case.max_q_len)
        self.shape = pk.attn_shape(self.q, self.k, self.bt, mq, case.scale, total_pages)
        self.shape.pages_per_split = pages_per_split
        if plan:   # the host-side plan from the lengths
            pk.pkv_attn_plan(self.shape, case.seq_lens)
        self.ws = pk.new_attn_workspace(self.shape)
        self.out = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")

    def run(self, stream=None):
        self.pk.pkv_attn_fwd(self.q, self.k, self.v, self.bt, self.sl, self.ql, self.out, self.shape,
                             self.ws, stream)
        return self.out

    def result(self):
        self.run()
        torch.cuda.synchronize()
        return self.out.cpu().numpy()

    def errors(self):
        return self.pk.pkv_attn_check_errors(self.ws)


def attn_gpu(case, pk, **kw):
    dc = DeviceCase(case, pk, **kw)
    out = dc.result()
    flags = dc.errors()
    return out, flags


def assert_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref32 = np.asarray(ref, dtype=np.float32).astype(np.float64)
    assert gpu.shape == ref32.shape, (gpu.shape, ref32.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref32)
    bound = TOL_ATOL + TOL_RTOL * np.abs(ref32)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside atol {TOL_ATOL} + rtol "
                             f"{TOL_RTOL}; worst at {i}: gpu {gpu[i]!r} oracle {ref32[i]!r}")
    return float(err.max())


def accept_gpu(acc, pk, window=True):
    logits = torch.from_numpy(np.ascontiguousarray(acc.logits)).cuda()
    drafts = dev_i32(acc.draft_ids) if acc.draft_ids.size else torch.empty(0, dtype=torch.int32,
                                                                           device="cuda")
    nd = dev_i32(acc.n_draft)
    B = acc.num_seqs
    oa = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    on = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    win = dev_i32(acc.window) if window else None
    shape = pk.accept_shape(logits, nd, acc.max_draft)
    ws = pk.new_accept_workspace(shape)
    pk.pkv_accept(logits, drafts, nd, oa, on, win, shape, ws)
    torch.cuda.synchronize()
    return oa.cpu().numpy(), on.cpu().numpy(), (win.cpu().numpy() if window else None)
