"""Configuration 5: a fragmented pool driven by a FIFO job queue.

Reading of the configuration (48 sequences of log-uniform length in
[256, 16384] "filling" a 256-page pool, which cannot hold them at once): the
jobs pass through a first-in-first-out queue as a continuous-batching
generator runs them. The pool first goes through seeded allocate/free churn by
"ghost" tenants, which leaves holes. Then, step by step:

1. admit queued jobs, in order, while the head job's pages fit; each admitted
   job takes the lowest free page indices (so new jobs fill holes) and its K/V
   is written into those pages;
2. the active batch (admission order) is verified in one pass;
3. the oldest active job retires and its pages return to the free list.

Ghost pages and freed pages hold bf16 NaN. The simulation is pure layout:
integer page bookkeeping plus seeded draws.
"""

from dataclasses import dataclass
import math

import numpy as np

from .bf16 import normal_bf16, BF16_QNAN
from .configs import PAGE, AttnCase, AcceptCase, _plant_drafts, _rng

CFG = 5


@dataclass
class Job:
    jid: int
    seq_len: int
    q_len: int
    pages: list = None


@dataclass
class Step:
    index: int
    case: AttnCase           # the active batch over the current pool
    accept: AcceptCase       # logits/drafts of the active jobs, packed in batch order
    job_ids: list            # job id of every batch row
    dirty_pages: np.ndarray  # pages whose content changed since the previous step


class Config5Queue:
    def __init__(self, seed=0, n_jobs=48, num_pages=256, Hq=32, Hkv=8, D=128, vocab=128256,
                 churn_ops=64, ghost_cap=64, table_width=64):
        self.seed, self.P, self.Hq, self.Hkv, self.D, self.vocab = seed, num_pages, Hq, Hkv, D, vocab
        self.table_width = table_width
        self.scale = float(np.float32(1.0 / math.sqrt(D)))
        lay = _rng(CFG, seed, 0)
        self.k_pool = np.full((num_pages, Hkv, PAGE, D), BF16_QNAN, dtype=np.uint16)
        self.v_pool = np.full((num_pages, Hkv, PAGE, D), BF16_QNAN, dtype=np.uint16)
        free = set(range(num_pages))
        ghosts = []
        occupancy = 0
        for _ in range(churn_ops):
            size = int(lay.integers(1, 17))
            want_free = ghosts and (lay.random() < 0.4 or occupancy + size > ghost_cap)
            if want_free:
                g = ghosts.pop(int(lay.integers(0, len(ghosts))))
                occupancy -= len(g)
                free.update(g)
            elif occupancy + size <= ghost_cap:
                pick = lay.choice(sorted(free), size, replace=False)
                ghosts.append([int(p) for p in pick])
                occupancy += size
                free.difference_update(ghosts[-1])
        self.ghost_pages = sorted(p for g in ghosts for p in g)
        self.free = free
        lo, hi = math.log(256), math.log(16384)
        self.jobs = []
        for j in range(n_jobs):
            L = int(math.floor(math.exp(lay.uniform(lo, hi))))
            L = min(max(L, 256), 16384)
            ql = int(lay.choice([1, 3, 5, 7]))
            self.jobs.append(Job(j, L, ql))
        self._job_data = {}

    # per-job draws, independent of when the job is admitted
    def _job_payload(self, job):
        if job.jid not in self._job_data:
            n = (job.seq_len + PAGE - 1) // PAGE
            shape = (n, self.Hkv, PAGE, self.D)
            k = normal_bf16(_rng(CFG, self.seed, 2, job.jid), shape)
            v = normal_bf16(_rng(CFG, self.seed, 3, job.jid), shape)
            tail = job.seq_len - (n - 1) * PAGE
            if tail < PAGE:
                k[n - 1, :, tail:, :] = BF16_QNAN
                v[n - 1, :, tail:, :] = BF16_QNAN
            q = normal_bf16(_rng(CFG, self.seed, 1, job.jid), (job.q_len, self.Hq, self.D))
            acc = _plant_drafts(_rng(CFG, self.seed, 4, job.jid), _rng(CFG, self.seed, 5, job.jid),
                                [job.q_len], self.vocab)
            self._job_data[job.jid] = (k, v, q, acc)
        return self._job_data[job.jid]

    def job_case(self, jid):
        """The job alone, over a private contiguous pool (for the oracle)."""
        job = self.jobs[jid]
        k, v, q, acc = self._job_payload(job)
        n = k.shape[0]
        table = np.arange(n, dtype=np.int32)[None, :]
        case = AttnCase(f"config5-job{jid}", q, k, v, table, np.array([job.seq_len], np.int32),
                        np.array([job.q_len], np.int32), self.scale)
        return case, acc

    def steps(self):
        queue = list(self.jobs)
        active = []
        free = set(self.free)
        dirty = set()
        step = 0
        while queue or active:
            while queue:
                need = (queue[0].seq_len + PAGE - 1) // PAGE
                if need > len(free):
                    break
                job = queue.pop(0)
                job.pages = sorted(free)[:need]
                free.difference_update(job.pages)
                k, v, _, _ = self._job_payload(job)
                self.k_pool[job.pages] = k
                self.v_pool[job.pages] = v
                dirty.update(job.pages)
                active.append(job)
            B = len(active)
            table = np.full((B, self.table_width), -1, dtype=np.int32)
            qs, logits, drafts, nd, match = [], [], [], [], []
            for b, job in enumerate(active):
                table[b, :len(job.pages)] = job.pages
                _, _, q, acc = self._job_payload(job)
                qs.append(q)
                logits.append(acc.logits)
                drafts.append(acc.draft_ids)
                nd.append(acc.n_draft)
                match.append(acc.planted_match)
            case = AttnCase(f"config5-step{step}", np.concatenate(qs), self.k_pool, self.v_pool, table,
                            np.array([j.seq_len for j in active], np.int32),
                            np.array([j.q_len for j in active], np.int32), self.scale,
                            meta={"cfg": 5, "seed": self.seed, "step": step})
            accept = AcceptCase(np.concatenate(logits), np.concatenate(drafts).astype(np.int32),
                                np.concatenate(nd).astype(np.int32), np.concatenate(match).astype(np.int32),
                                np.full(B, 5, np.int32))
            yield Step(step, case, accept, [j.jid for j in active],
                       np.array(sorted(dirty), dtype=np.int64))
            dirty = set()
            old = active.pop(0)
            free.update(old.pages)
            self.k_pool[old.pages] = BF16_QNAN
            self.v_pool[old.pages] = BF16_QNAN
            dirty.update(old.pages)
            step += 1
