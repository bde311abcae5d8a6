#!/usr/bin/env python3
"""Benchmark of the paged-attention + greedy-accept hot path on one MI355X.

A step is one speculative-verify pass over the verify workload: paged
attention for 8 sequences of 8192 cached tokens (window of 6 rows = 5 drafts +
1, causal inside the window; 32 q heads over 8 KV heads, head_dim 128, bf16,
256-token pages filling a 256-page pool through permuted block tables), then
the greedy accept over fp32 logits [48, 128256] with the window update. Inputs
are seeded synthetic data resident in HBM before timing; the K/V pools and
logits rotate over several replicas so that no step is served from the
256 MB last-level cache left warm by the previous one.

Prints one JSON line. `value` is the logical K/V bytes the step reads through
the block tables divided by the step time (attention + accept); the line also
carries the attention-only rate, the HBM fraction, verified tokens/s, the
roofline of the attention kernel, per-configuration attention rates for the
decode and dedup workloads, and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, AMD's published figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core rate, AMD's published figure
METRIC = "paged-attn KV read GB/s (fraction of HBM peak); verified tokens/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration sweep")
    ap.add_argument("--no-prefill", action="store_true", help="skip the long-window (prefill) leg")
    ap.add_argument("--no-queue", action="store_true", help="skip the mixed job-queue leg")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the CPU oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run device-to-device copies of a known size (the reference dispatches "
                         "that scale the rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes)")
    return ap.parse_args()


# Sources of the attention kernel: a stored HBM-traffic measurement is used only
# while their hash matches the one recorded with it.
KERNEL_SOURCES = ("paged_kv_attention_attn_amd/csrc/attn_kernels.hip", "paged_kv_attention_attn_amd/csrc/device.h",
                  "paged_kv_attention_attn_amd/csrc/internal.h")
TRAFFIC_PROFILE = "profiles/attn_split_kernel_mfma.verify_8x8192_w6.md"
DEDUP_PROFILE = "profiles/attn_split_kernel_valu.dedup_100x4096_shared.md"   # configuration 4, plain call
COPY_CAL_BYTES = 256 << 20


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(profile=TRAFFIC_PROFILE):
    """HBM bytes per launch of an attention kernel from its committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by its
    reading on a plain copy of known size), or None when the summary is
    missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, profile)
    try:
        text = open(path).read()
        block = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(block)
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec


def copy_calibration(torch):
    """Device-to-device copies of COPY_CAL_BYTES each: the plain copy kernel
    whose counter readings calibrate FETCH_SIZE and WRITE_SIZE."""
    src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    n = 5
    for _ in range(n):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_CAL_BYTES, "copies": n}), flush=True)


class Attn:
    """One attention workload on the device, with R replicas of its pools."""

    def __init__(self, case, pk, torch, replicas):
        self.case, self.pk, self.torch = case, pk, torch
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        k0, v0 = dev(case.k_pool), dev(case.v_pool)
        self.k = [k0] + [k0.clone() for _ in range(replicas - 1)]
        self.v = [v0] + [v0.clone() for _ in range(replicas - 1)]
        self.q = dev(case.q)
        self.bt, self.sl, self.ql = i32(case.block_table), i32(case.seq_lens), i32(case.q_lens)
        self.out = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
        # the host knows the lengths: they plan the splits
        self.shape = pk.pkv_attn_plan(pk.attn_shape(self.q, k0, self.bt, max(1, case.max_q_len), case.scale),
                                      case.seq_lens)
        self.ws = pk.new_attn_workspace(self.shape)
        self.R = replicas

    def __call__(self, i):
        r = i % self.R
        self.pk.pkv_attn_fwd(self.q, self.k[r], self.v[r], self.bt, self.sl, self.ql, self.out,
                             self.shape, self.ws)


class Accept:
    def __init__(self, acc, pk, torch, replicas):
        self.pk, self.torch = pk, torch
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        l0 = torch.from_numpy(np.ascontiguousarray(acc.logits)).cuda()
        self.logits = [l0] + [l0.clone() for _ in range(replicas - 1)]
        self.drafts = i32(acc.draft_ids)
        self.nd = i32(acc.n_draft)
        self.oa = torch.empty(acc.num_seqs, dtype=torch.int32, device="cuda")
        self.on = torch.empty(acc.num_seqs, dtype=torch.int32, device="cuda")
        self.win0 = i32(acc.window)
        self.win = self.win0.clone()
        self.shape = pk.accept_shape(l0, self.nd, acc.max_draft)
        self.ws = pk.new_accept_workspace(self.shape)
        self.R = replicas

    def __call__(self, i):
        self.pk.pkv_accept(self.logits[i % self.R], self.drafts, self.nd, self.oa, self.on, self.win,
                           self.shape, self.ws)


QUANT = {  # format: (encode call, attention call, code dtype, code bytes per value)
    "q8": ("pkv_q8_encode", "pkv_attn_fwd_q8", "int8", 1.0),
    "q4": ("pkv_q4_encode", "pkv_attn_fwd_q4", "uint8", 0.5),
}


def quant_codes(torch, pk, fmt, k, v):
    """Encode bf16 pools k, v into (k codes, k scales, v codes, v scales) on the GPU."""
    enc, _, dt, per = QUANT[fmt]
    P, Hkv, page, D = k.shape
    out = []
    for x in (k, v):
        c = torch.empty(P, Hkv, page, int(D * per), dtype=getattr(torch, dt), device="cuda")
        sc = torch.empty(P, Hkv, page, dtype=torch.float32, device="cuda")
        getattr(pk, enc)(x, c, sc)
        out += [c, sc]
    return out


def quant_leg(torch, pk, seed, R, steps, warmup, bf16_us):
    """Attention over the quantized caches (Q8: int8 codes, Q4: two 4-bit
    codes per byte, each with one fp32 scale per token and KV head) on the
    batched-decode and verify workloads: the pools are encoded on the GPU by
    the library's encoders, then timed like the bf16 calls (R replicas)."""
    from workloads import make_config
    res = {"q8": {}, "q4": {}}
    for cfg in (2, 3):
        c, _ = make_config(cfg, seed=seed)
        a = Attn(c, pk, torch, 1)
        D = c.head_dim
        tokens = int(np.sum(c.seq_lens, dtype=np.int64))
        for fmt in ("q8", "q4"):
            log(f"{fmt} cache, configuration {cfg}")
            reps = [quant_codes(torch, pk, fmt, a.k[0], a.v[0])]
            reps += [[t.clone() for t in reps[0]] for _ in range(R - 1)]
            call = getattr(pk, QUANT[fmt][1])
            f = lambda i: call(a.q, *reps[i % R], a.bt, a.sl, a.ql, a.out, a.shape, a.ws)
            ms = time_ms(torch, f, steps, warmup)
            assert pk.pkv_attn_check_errors(a.ws) == 0, f"{fmt} attention flagged its inputs"
            qb = int(tokens * c.num_kv_heads * 2 * (D * QUANT[fmt][3] + 4))
            res[fmt][f"config{cfg}"] = {
                "attn_us": round(ms * 1e3, 3), "code_bytes": qb, "code_gbps": round(qb / (ms * 1e-3) / 1e9, 2),
                "hbm_fraction": round(qb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "speedup_vs_bf16": round(bf16_us[cfg] / (ms * 1e3), 3) if cfg in bf16_us else None,
                "decode_tokens_per_s": round(c.num_seqs / (ms * 1e-3), 1)}
            del reps
            torch.cuda.empty_cache()
        del a
        torch.cuda.empty_cache()
    # a decode batch long enough that streaming the cache sets the time:
    # 16 sequences x 32768 tokens (2.1 GB of bf16 K/V, far above the caches),
    # pools drawn on the GPU, the same call sequence for every format
    B, L, Hq, Hkv, D = 16, 32768, 32, 8, 128
    log("quantized caches, long decode batch")
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    npg, P = L // 256, B * (L // 256) + 8
    k = torch.randn(P, Hkv, 256, D, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(P, Hkv, 256, D, device="cuda", generator=g).to(torch.bfloat16)
    table = torch.randperm(P, device="cuda", generator=g)[:B * npg].to(torch.int32).view(B, npg).contiguous()
    sl = torch.full((B,), L, dtype=torch.int32, device="cuda")
    ql = torch.ones(B, dtype=torch.int32, device="cuda")
    q = torch.randn(B, Hq, D, device="cuda", generator=g).to(torch.bfloat16)
    out = torch.empty(B, Hq, D, device="cuda")
    shape = pk.pkv_attn_plan(pk.attn_shape(q, k, table, 1, D ** -0.5), np.full(B, L, np.int32))
    ws = pk.new_attn_workspace(shape)
    tb = time_ms(torch, lambda i: pk.pkv_attn_fwd(q, k, v, table, sl, ql, out, shape, ws), steps, warmup)
    kvb = B * L * Hkv * D * 4
    long = {"bf16_us": round(tb * 1e3, 2), "bf16_gbps": round(kvb / tb / 1e6, 1),
            "bf16_hbm_fraction": round(kvb / tb / 1e6 / HBM_PEAK_GBPS, 4)}
    for fmt in ("q8", "q4"):
        codes = quant_codes(torch, pk, fmt, k, v)
        call = getattr(pk, QUANT[fmt][1])
        tq = time_ms(torch, lambda i: call(q, *codes, table, sl, ql, out, shape, ws), steps, warmup)
        assert pk.pkv_attn_check_errors(ws) == 0
        qb = int(B * L * Hkv * 2 * (D * QUANT[fmt][3] + 4))
        long.update({f"{fmt}_us": round(tq * 1e3, 2), f"{fmt}_code_gbps": round(qb / tq / 1e6, 1),
                     f"{fmt}_speedup_vs_bf16": round(tb / tq, 3)})
        del codes
        torch.cuda.empty_cache()
    res["long_decode_16x32768"] = long
    del k, v
    torch.cuda.empty_cache()
    return res


def time_ms(torch, fn, steps, warmup):
    """Mean milliseconds per call of fn(i), timed with HIP events on the
    current stream (the stream every launch goes to)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def launch_percentiles(torch, fn, steps, warmup):
    """Median, p10 and p90 microseconds of single calls of fn(i), each
    bracketed by its own pair of HIP events on the current stream."""
    for i in range(warmup):
        fn(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(warmup + i)
        b.record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    return {"median": round(float(np.median(us)), 3), "p10": round(float(np.percentile(us, 10)), 3),
            "p90": round(float(np.percentile(us, 90)), 3)}


def cache_leg(torch, pk, case, attn, accept, steps, warmup):
    """The cache calls around the verify pass on the same workload: append the
    window's K/V (sequences hold seq_len - q_len tokens before it), and roll
    back with accepted = 0, which restores the state so every repetition is
    the same work. Also one whole loop step: append, attention, accept,
    rollback (to the same restored state)."""
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    B, rows = case.num_seqs, int(case.q_lens.sum())
    Hkv, D = case.num_kv_heads, case.head_dim
    rng = np.random.default_rng(1)
    k_new = torch.from_numpy(rng.integers(0x3C00, 0x3F80, (rows, Hkv, D), dtype=np.uint16).view(np.int16)) \
        .view(torch.bfloat16).cuda()
    v_new = k_new.clone()
    before = i32(case.seq_lens - case.q_lens)
    lens = before.clone()
    free = i32(np.full(case.k_pool.shape[0], -1))
    count = i32([0])
    zeros = i32(np.zeros(B))
    shape = pk.kv_shape(attn.k[0], attn.bt, rows)
    ws = pk.new_kv_workspace(shape)

    def append_rollback(i):
        r = i % attn.R
        pk.pkv_kv_append(k_new, v_new, attn.k[r], attn.v[r], attn.bt, lens, attn.ql, free, count, shape, ws)
        pk.pkv_kv_rollback(attn.bt, lens, attn.ql, zeros, free, count, shape, ws)

    def loop_step(i):
        r = i % attn.R
        pk.pkv_kv_append(k_new, v_new, attn.k[r], attn.v[r], attn.bt, lens, attn.ql, free, count, shape, ws)
        pk.pkv_attn_fwd(attn.q, attn.k[r], attn.v[r], attn.bt, lens, attn.ql, attn.out, attn.shape, attn.ws)
        accept(i)
        pk.pkv_kv_rollback(attn.bt, lens, attn.ql, zeros, free, count, shape, ws)

    pair_ms = time_ms(torch, append_rollback, steps, warmup)
    loop_ms = time_ms(torch, loop_step, steps, warmup)
    torch.cuda.synchronize()
    assert torch.equal(lens, before), "append + rollback(0) must restore the lengths"
    assert pk.pkv_kv_check_errors(ws) == 0
    return {"append_rollback_us": round(pair_ms * 1e3, 3), "verify_loop_step_us": round(loop_ms * 1e3, 3),
            "window_kv_bytes_written": rows * Hkv * D * 2 * 2,
            "note": "append writes the window's K/V (q_len rows per sequence); rollback with accepted = 0 "
                    "restores the state; the loop step is append + attention + accept + rollback"}


def prefill_flops(case):
    """Algorithmic flops of a long-window pass: every window row of every q
    head does 2 * D multiply-adds per visible key for q.k and as many for p.v
    (4 * D flops); row i of a q_len window over seq_len cached tokens sees
    seq_len - q_len + i + 1 keys. Padding rows and masked keys are not counted."""
    tot = 0
    for L, ql in zip(case.seq_lens, case.q_lens):
        L, ql = int(L), int(ql)
        tot += ql * (L - ql) + ql * (ql + 1) // 2
    return tot * case.num_q_heads * 4 * case.head_dim


def prefill_leg(torch, pk, seed, steps, warmup):
    """The long-window kernel on two prefill workloads: the verify
    configuration's cache as a whole-prompt prefill (8 x 8192 tokens), and
    the prefix-dedup layout prefilling only each sequence's private tail over
    the shared 4096-token prefix. Rates are algorithmic bf16 flops against
    the dense bf16 matrix-core peak."""
    from workloads import make_prefill_config
    out = {}
    for which in ("full", "dedup"):
        log(f"prefill {which}")
        c = make_prefill_config(which, seed=seed)
        a = Attn(c, pk, torch, 1)
        ms = time_ms(torch, a, steps, warmup)
        pct = launch_percentiles(torch, a, steps, warmup)
        torch.cuda.synchronize()
        assert pk.pkv_attn_check_errors(a.ws) == 0
        fl = prefill_flops(c)
        tflops = fl / (ms * 1e-3) / 1e12
        out[which] = {"us": round(ms * 1e3, 1), "us_per_launch": pct, "flops": int(fl),
                      "tflops": round(tflops, 1), "mfma_fraction": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                      "tokens_per_s": round(float(c.q_lens.sum()) / (ms * 1e-3), 1),
                      "window_tokens": int(c.q_lens.sum()), "cached_tokens": int(c.seq_lens.sum())}
        if which == "dedup":
            # the same tails through the shared-prefix call: every tail row of
            # the batch stacked against the 16 shared pages once per KV head,
            # then each tail over its own keys, merged by log-sum-exp
            log("prefill dedup through the shared-prefix call")
            shared = 16
            ws = pk.new_attn_shared_workspace(a.shape, shared)
            f = lambda i: pk.pkv_attn_fwd_shared(a.q, a.k[0], a.v[0], a.bt, a.sl, a.ql, a.out, a.shape, shared, ws)
            a(0)
            torch.cuda.synchronize()
            plain = a.out.cpu().numpy()
            ms_s = time_ms(torch, f, steps, warmup)
            torch.cuda.synchronize()
            assert pk.pkv_attn_check_errors(ws) == 0, "shared-prefix call flagged its inputs"
            got = a.out.cpu().numpy()
            # both calls meet the oracle's tolerance, so they agree within twice it
            assert np.all(np.abs(got - plain) <= 2 * (2e-3 + 1e-2 * np.abs(plain))), "shared call != plain call"
            tf_s = fl / (ms_s * 1e-3) / 1e12
            out[which]["shared_call"] = {
                "us": round(ms_s * 1e3, 1), "tflops": round(tf_s, 1),
                "mfma_fraction": round(tf_s / MFMA_BF16_PEAK_TFLOPS, 4), "shared_pages": shared,
                "note": "pkv_attn_fwd_shared on the same batch (same algorithmic flops); output checked "
                        "against the plain call"}
            del ws
        del a
        torch.cuda.empty_cache()
    out["note"] = ("algorithmic flops = 4 * head_dim * q_heads * sum over window rows of visible keys; "
                   "peak = dense bf16 matrix-core rate")
    return out


def queue_leg(torch, pk, seed, steps, warmup):
    """The mixed job queue (48 jobs of 256..16384 tokens with windows of 1, 3,
    5 or 7 rows, admitted into a churned 256-page pool as pages free up, the
    oldest retiring each step): every step's attention and accept timed on
    its own inputs (HIP events, replicated pools not needed: the steps differ).
    Verified tokens/s = accepted tokens over the summed attention + accept time."""
    from workloads import Config5Queue, kv_logical_bytes
    q = Config5Queue(seed=seed)
    t_attn = t_acc = 0.0
    accepted = kv = n = rows = 0
    for st in q.steps():
        c = st.case
        a = Attn(c, pk, torch, 1)
        ac = Accept(st.accept, pk, torch, 1)
        t_attn += time_ms(torch, a, steps, warmup)
        t_acc += time_ms(torch, ac, steps, warmup)
        ac.win.copy_(ac.win0)
        a(0)
        ac(0)
        torch.cuda.synchronize()
        assert pk.pkv_attn_check_errors(a.ws) == 0, f"queue step {st.index}: attention error flags"
        got = ac.oa.cpu().numpy()
        assert np.array_equal(got, st.accept.planted_match + 1), f"queue step {st.index}: accepted counts"
        accepted += int(got.sum())
        kv += kv_logical_bytes(c.seq_lens, c.num_kv_heads, c.head_dim)
        rows += int(c.q_lens.sum())
        n += 1
        del a, ac
    torch.cuda.empty_cache()
    return {"steps": n, "window_rows": rows, "accepted_tokens": accepted, "kv_bytes": kv,
            "attn_us_total": round(t_attn * 1e3, 2), "accept_us_total": round(t_acc * 1e3, 2),
            "kv_gbps": round(kv / (t_attn * 1e-3) / 1e9, 2),
            "verified_tokens_per_s": round(accepted / ((t_attn + t_acc) * 1e-3), 1),
            "note": "single layer, no model GEMMs; accepted counts checked against the planted draft matches"}


def pool_leg(torch, pk, steps, warmup):
    """The page allocator: host admissions of the prefix-dedup job mix (100
    prompts of a shared 4096-token prefix plus a private tail of 1..256
    tokens into a 256-page pool: page lookups by prefix, reference counts),
    and the device side of a defragmentation, page copies of the verify
    configuration's pools (8 KV heads x 256 x 128, K and V: 1 MiB a page),
    timed on 128 disjoint moves."""
    rng = np.random.default_rng(4)
    prefix = rng.integers(0, 128000, 4096).tolist()
    prompts = [np.array(prefix + rng.integers(0, 128000, int(rng.integers(1, 257))).tolist(), np.int32)
               for _ in range(100)]
    tokens = sum(len(p) for p in prompts)
    reps = 5
    t0 = time.perf_counter()
    for _ in range(reps):
        pool = pk.pkv_pool_create(256)
        held = [pk.pkv_pool_admit(pool, p)[0] for p in prompts]
        for pages in held:
            pk.pkv_pool_release(pool, pages)
        pk.pkv_pool_destroy(pool)
    host_s = (time.perf_counter() - t0) / reps
    P, Hkv, D, n = 256, 8, 128, 128
    k = torch.empty((P, Hkv, 256, D), dtype=torch.bfloat16, device="cuda").normal_()
    v = torch.empty_like(k).normal_()
    src = torch.arange(P - n, P, dtype=torch.int32, device="cuda")
    dst = torch.arange(0, n, dtype=torch.int32, device="cuda")
    ms = time_ms(torch, lambda i: pk.pkv_pool_copy_pages(k, v, src, dst), steps, warmup)
    moved = n * 2 * Hkv * 256 * D * 2
    gbps = 2 * moved / (ms * 1e-3) / 1e9
    del k, v
    torch.cuda.empty_cache()
    return {"admit_release_us_per_job": round(host_s / len(prompts) * 1e6, 2),
            "host_tokens_per_s": round(tokens / host_s, 1),
            "copy_pages_us": round(ms * 1e3, 2), "bytes_moved": moved,
            "copy_gbps": round(gbps, 1), "copy_hbm_fraction": round(gbps / HBM_PEAK_GBPS, 4),
            "note": "host: admit + release per job of the dedup mix (every job after the first reuses the "
                    "16 prefix pages); device: 128 page moves, traffic = 2 x bytes moved"}


def cpu_baseline(case, acc, seconds):
    """The CPU oracle on the verify step: whole sequences (attention over
    their cached tokens + accept over their logits rows) in order, passes
    over the batch repeated until the time budget is spent (at least one
    sequence)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    kv_per_tok = 2 * case.num_kv_heads * case.head_dim * 2
    done_seqs, kv_bytes, accepted = 0, 0, 0
    t0 = time.perf_counter()
    while True:
        r0 = 0
        for b in range(case.num_seqs):
            ql = int(case.q_lens[b])
            oracle.attention(case.q[r0:r0 + ql], case.k_pool, case.v_pool, case.block_table[b:b + 1],
                             case.seq_lens[b:b + 1], case.q_lens[b:b + 1], case.scale)
            nd = acc.n_draft[b:b + 1]
            d0 = int(acc.n_draft[:b].sum())
            a, _, _ = oracle.accept(acc.logits[r0:r0 + ql], acc.draft_ids[d0:d0 + int(nd[0])], nd)
            accepted += int(a[0])
            kv_bytes += int(case.seq_lens[b]) * kv_per_tok
            done_seqs += 1
            r0 += ql
            if time.perf_counter() - t0 > seconds:
                break
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": kv_bytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{done_seqs} sequence passes ({done_seqs / case.num_seqs:.2f} x the {case.num_seqs}-sequence "
                      f"verify batch): float64 attention over {int(case.seq_lens[0])} cached tokens x "
                      f"{int(case.q_lens[0])} window rows x {case.num_q_heads} heads, plus accept over each "
                      f"sequence's {acc.vocab}-wide logits rows; {dt:.1f} s",
            "verified_tokens_per_s": accepted / dt, "seconds": dt,
            "host_cores_available": len(os.sched_getaffinity(0)), "cpu_model": cpu}


def roofline(kv_bytes, attn_ms):
    """Roofline of the attention kernel on the verify workload: algorithmic
    K/V bytes per launch over the mean launch time measured above, against
    the HBM peak; `traffic` is the measured HBM bytes per launch."""
    achieved = kv_bytes / (attn_ms * 1e-3) / 1e9
    rec = stored_traffic()
    traffic = None if rec is None else int(rec["hbm_bytes_per_launch"])
    return {"bound": "hbm", "kernel": "attn_split_kernel<128, MfmaTile<128, 1>, 2, 4>",
            "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "traffic_gbps": None if traffic is None else round(traffic / (attn_ms * 1e-3) / 1e9, 2),
            "traffic_profile": TRAFFIC_PROFILE if rec is not None else None,
            "algorithmic_bytes_per_launch": kv_bytes,
            "avg_launch_us": round(attn_ms * 1e3, 3)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path: the hot path shards by sequence and KV head with no exchange", flush=True)
        sys.exit(2)

    import torch
    import paged_kv_attention_attn_amd as pk
    from workloads import make_config, kv_logical_bytes

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    props = torch.cuda.get_device_properties(0)
    R = max(1, args.replicas)

    log("generating the verify workload")
    case, acc = make_config(3, seed=args.seed)
    attn = Attn(case, pk, torch, R)
    accept = Accept(acc, pk, torch, R)
    kv_bytes = kv_logical_bytes(case.seq_lens, case.num_kv_heads, case.head_dim)

    def step(i):
        attn(i)
        accept(i)

    log("timing")
    attn_ms = time_ms(torch, attn, args.steps, args.warmup)
    accept_ms = time_ms(torch, accept, args.steps, args.warmup)
    accept.win.copy_(accept.win0)
    torch.cuda.synchronize()
    step_ms = time_ms(torch, step, args.steps, args.warmup)
    attn_pct = launch_percentiles(torch, attn, args.steps, args.warmup)
    accept.win.copy_(accept.win0)
    accept_pct = launch_percentiles(torch, accept, args.steps, args.warmup)
    # one checked step: the window update is applied per call, so reset and run once
    accept.win.copy_(accept.win0)
    step(0)
    torch.cuda.synchronize()
    accepted = int(accept.oa.sum().item())
    flags = pk.pkv_attn_check_errors(attn.ws)
    assert flags == 0, f"attention error flags {flags}"

    value = kv_bytes / (step_ms * 1e-3) / 1e9
    attn_gbps = kv_bytes / (attn_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "speculative verify: 8 sequences x 8192 cached tokens, window 6 (5 drafts + 1) "
                               "causal inside the window, 32 q / 8 KV heads, head_dim 128, bf16 K/V in "
                               "256-token pages (full 256-page pool, permuted tables), then greedy accept "
                               "over fp32 logits [48, 128256] with the +2/-1 window rule",
                   "global_batch": int(case.num_seqs), "seq_len": int(case.seq_lens[0]),
                   "q_len": int(case.q_lens[0]), "parallelism": "single GPU"},
        "value_note": "value = K/V bytes per step / (attention + accept) time per step; "
                      "attn_kv_gbps and roofline are the attention kernel alone",
        "hbm_fraction": round(value / HBM_PEAK_GBPS, 4),
        "attn_kv_gbps": round(attn_gbps, 2),
        "attn_hbm_fraction": round(attn_gbps / HBM_PEAK_GBPS, 4),
        "attn_us": round(attn_ms * 1e3, 3),
        "accept_us": round(accept_ms * 1e3, 3),
        "attn_us_per_launch": attn_pct,
        "accept_us_per_call": accept_pct,
        "verified_tokens_per_s": round(accepted / (step_ms * 1e-3), 1),
        "accepted_per_step": accepted,
        "kv_bytes_per_step": kv_bytes,
        "roofline": roofline(kv_bytes, attn_ms),
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count, "hbm_gib": round(props.total_memory / 2**30, 1)},
    }
    log("cache append / rollback")
    accept.win.copy_(accept.win0)
    result["cache"] = cache_leg(torch, pk, case, attn, accept, args.steps, args.warmup)
    del attn, accept
    torch.cuda.empty_cache()

    if not args.no_configs:
        sweep = {}
        for cfg in (1, 2, 4):
            log(f"configuration {cfg}")
            c, ca = make_config(cfg, seed=args.seed)
            a = Attn(c, pk, torch, R)
            ms = time_ms(torch, a, args.steps, args.warmup)
            kb = kv_logical_bytes(c.seq_lens, c.num_kv_heads, c.head_dim)
            ent = {"attn_us": round(ms * 1e3, 3), "kv_bytes": kb,
                   "kv_gbps": round(kb / (ms * 1e-3) / 1e9, 2),
                   "hbm_fraction": round(kb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                   "decode_tokens_per_s": round(c.num_seqs / (ms * 1e-3), 1)}
            if cfg == 4:
                # shared prefix pages are read through one L2 per XCD, so the
                # logical K/V bytes (the prefix counted once per sequence) far
                # exceed what DRAM delivers: a logical rate, not an HBM fraction
                ent["kv_bytes_logical"] = ent.pop("kv_bytes")
                ent["kv_gbps_logical"] = ent.pop("kv_gbps")
                ent["logical_rate_over_hbm_peak"] = ent.pop("hbm_fraction")
                rec = stored_traffic(DEDUP_PROFILE)
                ent["dram_bytes_per_launch"] = None if rec is None else int(rec["hbm_bytes_per_launch"])
                ent["dram_gbps"] = None if rec is None else round(rec["hbm_bytes_per_launch"] / (ms * 1e-3) / 1e9, 2)
                ent["dram_profile"] = DEDUP_PROFILE if rec is not None else None
            sweep[f"config{cfg}"] = ent
            if ca is not None:   # a verify step: attention + accept
                ac = Accept(ca, pk, torch, R)
                ms_acc = time_ms(torch, ac, args.steps, args.warmup)
                ac.win.copy_(ac.win0)
                ac(0)
                torch.cuda.synchronize()
                got = int(ac.oa.sum().item())
                sweep[f"config{cfg}"].update({"accept_us": round(ms_acc * 1e3, 3), "accepted_per_step": got,
                                              "verified_tokens_per_s": round(got / ((ms + ms_acc) * 1e-3), 1)})
                del ac
            torch.cuda.empty_cache()
        log("configuration 4 through the shared-prefix call")
        c, _ = make_config(4, seed=args.seed)
        a = Attn(c, pk, torch, R)
        shared = 16   # every table of the dedup workload starts with the same 16 pages
        ws = pk.new_attn_shared_workspace(a.shape, shared)
        f = lambda i: pk.pkv_attn_fwd_shared(a.q, a.k[i % R], a.v[i % R], a.bt, a.sl, a.ql, a.out, a.shape,
                                              shared, ws)
        ms = time_ms(torch, f, args.steps, args.warmup)
        assert pk.pkv_attn_check_errors(ws) == 0, "shared-prefix call flagged its inputs"
        kb = kv_logical_bytes(c.seq_lens, c.num_kv_heads, c.head_dim)
        sweep["config4_shared"] = {"attn_us": round(ms * 1e3, 3), "kv_bytes": kb,
                                   "kv_gbps_logical": round(kb / (ms * 1e-3) / 1e9, 2),
                                   "shared_pages": shared,
                                   "decode_tokens_per_s": round(c.num_seqs / (ms * 1e-3), 1),
                                   "note": "pkv_attn_fwd_shared: the shared prefix is attended once per KV "
                                           "head for all 400 window rows, the tails by the decode kernel"}
        del a, ws
        torch.cuda.empty_cache()
        sweep["config3"] = {"attn_us": result["attn_us"], "kv_bytes": kv_bytes,
                            "kv_gbps": result["attn_kv_gbps"], "hbm_fraction": result["attn_hbm_fraction"]}
        result["configs"] = sweep

    bf16_us = {3: result["attn_us"]}
    if "configs" in result:
        bf16_us[2] = result["configs"]["config2"]["attn_us"]
    result["quantized"] = quant_leg(torch, pk, args.seed, R, args.steps, args.warmup, bf16_us)

    if not args.no_queue:
        log("mixed job queue")
        result["queue"] = queue_leg(torch, pk, args.seed, max(5, args.steps // 5), max(2, args.warmup // 2))
    if not args.no_prefill:
        result["prefill"] = prefill_leg(torch, pk, args.seed, max(5, args.steps // 5), max(2, args.warmup // 2))
    log("page allocator")
    result["pool"] = pool_leg(torch, pk, args.steps, args.warmup)

    if not args.no_cpu_baseline:
        log("CPU oracle sample")
        result["cpu_baseline"] = cpu_baseline(case, acc, args.cpu_seconds)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
