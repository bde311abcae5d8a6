"""Seeded synthetic workloads: the five paged-attention configurations plus
small random cases and layout transforms used by the invariance tests.

Seeds follow ``np.random.SeedSequence([cfg, seed, stream])`` with streams
0 = layout / lengths / tables, 1 = Q, 2 = K, 3 = V, 4 = logits, 5 = drafts.

Q, K and V are float32 N(0, 1) rounded to bf16 (nearest-even). Pages that no
sequence references, and the slots of a sequence's last page past its length,
are filled with bf16 quiet NaN unless ``poison=False``: the attention result
must not depend on them.

Drafts for the speculative-verify cases are built by *planting*: a row whose
draft must match gets one logit set to ``PLANT`` (far above any N(0, 1) draw)
at a freshly drawn token id, and the draft is that id; the first row that must
mismatch is planted the same way and its draft is a different id. The generator
therefore knows the intended accepted length without evaluating any argmax.
"""

from dataclasses import dataclass, field
import math

import numpy as np

from .bf16 import f32_to_bf16_bits, normal_bf16, BF16_QNAN

PAGE = 256            # tokens per page; the pages fix it at 256
PLANT = np.float32(64.0)
INITIAL_WINDOW = 5    # first draft window of the assisted-generation loop


def _rng(cfg, seed, stream, *extra):
    return np.random.default_rng(np.random.SeedSequence([cfg, seed, stream, *extra]))


def _normal_bf16(rng, shape):
    return normal_bf16(rng, shape)


def _pages_for(seq_len):
    return (int(seq_len) + PAGE - 1) // PAGE


@dataclass
class AttnCase:
    name: str
    q: np.ndarray            # uint16 [total_q, Hq, D]
    k_pool: np.ndarray       # uint16 [P, Hkv, 256, D]
    v_pool: np.ndarray       # uint16 [P, Hkv, 256, D]
    block_table: np.ndarray  # int32 [B, W]
    seq_lens: np.ndarray     # int32 [B]
    q_lens: np.ndarray       # int32 [B]
    scale: float             # a float32-representable value
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return int(self.seq_lens.shape[0])

    @property
    def num_q_heads(self):
        return int(self.q.shape[1])

    @property
    def num_kv_heads(self):
        return int(self.k_pool.shape[1])

    @property
    def head_dim(self):
        return int(self.q.shape[2])

    @property
    def num_pages(self):
        return int(self.k_pool.shape[0])

    @property
    def max_pages_per_seq(self):
        return int(self.block_table.shape[1])

    @property
    def total_q(self):
        return int(self.q.shape[0])

    @property
    def max_q_len(self):
        return int(self.q_lens.max()) if self.q_lens.size else 1


@dataclass
class AcceptCase:
    logits: np.ndarray         # float32 [sum(n_draft + 1), V]
    draft_ids: np.ndarray      # int32 [sum(n_draft)]
    n_draft: np.ndarray        # int32 [B]
    planted_match: np.ndarray  # int32 [B]: index of the planted first mismatch (n = none)
    window: np.ndarray         # int32 [B]: draft window before this verify step

    @property
    def num_seqs(self):
        return int(self.n_draft.shape[0])

    @property
    def vocab(self):
        return int(self.logits.shape[1])

    @property
    def total_rows(self):
        return int(self.logits.shape[0])

    @property
    def max_draft(self):
        return int(self.n_draft.max()) if self.n_draft.size else 0


def kv_logical_bytes(seq_lens, num_kv_heads, head_dim):
    """K+V bytes attention reads through the block tables: valid tokens only."""
    return int(np.sum(seq_lens, dtype=np.int64)) * 2 * num_kv_heads * head_dim * 2


def _poison(k_pool, v_pool, block_table, seq_lens, poison):
    """NaN-fill unreferenced pages and the slots of last pages past every
    referencing sequence's length (a shared page keeps its longest valid run)."""
    if not poison:
        return
    P = k_pool.shape[0]
    valid = np.zeros(P, dtype=np.int64)
    for b in range(len(seq_lens)):
        for j in range(_pages_for(seq_lens[b])):
            p = int(block_table[b, j])
            valid[p] = max(valid[p], min(PAGE, int(seq_lens[b]) - j * PAGE))
    k_pool[valid == 0] = BF16_QNAN
    v_pool[valid == 0] = BF16_QNAN
    for p in np.nonzero((valid > 0) & (valid < PAGE))[0]:
        k_pool[p, :, valid[p]:, :] = BF16_QNAN
        v_pool[p, :, valid[p]:, :] = BF16_QNAN


def _q_for(rng, q_lens, Hq, D):
    return _normal_bf16(rng, (int(np.sum(q_lens)), Hq, D))


def _plant_drafts(rng_logits, rng_draft, q_lens, vocab):
    """Logits N(0,1) with planted maxima so that sequence b's first mismatch
    sits at a drawn index m_b in 0..n_b (m_b = n_b means every draft matches)."""
    q_lens = np.asarray(q_lens, dtype=np.int64)
    n_draft = (q_lens - 1).astype(np.int32)
    rows = int(q_lens.sum())
    logits = rng_logits.standard_normal(size=(rows, vocab), dtype=np.float32)
    drafts = np.zeros(int(n_draft.sum()), dtype=np.int32)
    match = np.zeros(len(q_lens), dtype=np.int32)
    r0 = 0
    d0 = 0
    for b, n in enumerate(n_draft):
        n = int(n)
        m = int(rng_draft.integers(0, n + 1))
        match[b] = m
        for i in range(n):
            if i < m:
                w = int(rng_draft.integers(0, vocab))
                logits[r0 + i, w] = PLANT
                drafts[d0 + i] = w
            elif i == m:
                w = int(rng_draft.integers(0, vocab))
                logits[r0 + i, w] = PLANT
                drafts[d0 + i] = (w + 1 + int(rng_draft.integers(0, vocab - 1))) % vocab
            else:
                drafts[d0 + i] = int(rng_draft.integers(0, vocab))
        r0 += n + 1
        d0 += n
    window = np.full(len(q_lens), INITIAL_WINDOW, dtype=np.int32)
    return AcceptCase(logits, drafts, n_draft, match, window)


def make_accept_case(seed, q_lens, vocab, cfg=100):
    """Accept-only case: sequence b verifies q_lens[b] rows (n_draft = q_len - 1)."""
    return _plant_drafts(_rng(cfg, seed, 4), _rng(cfg, seed, 5), q_lens, vocab)


def make_tiny_case(seed, seq_lens, q_lens, Hq=4, Hkv=2, D=64, num_pages=None,
                   table_width=None, poison=True, scale=None, name="tiny", cfg=99):
    """Random small case: each sequence gets distinct pages from a random
    permutation of the pool; spare pool pages stay unreferenced."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    B = len(seq_lens)
    pages = [_pages_for(s) for s in seq_lens]
    need = int(sum(pages))
    P = num_pages if num_pages is not None else need + 3
    assert P >= need
    W = table_width if table_width is not None else max(1, max(pages) if pages else 1)
    lay = _rng(cfg, seed, 0)
    perm = lay.permutation(P)
    table = np.full((B, W), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        table[b, :pages[b]] = perm[o:o + pages[b]]
        o += pages[b]
    q = _q_for(_rng(cfg, seed, 1), q_lens, Hq, D)
    k = _normal_bf16(_rng(cfg, seed, 2), (P, Hkv, PAGE, D))
    v = _normal_bf16(_rng(cfg, seed, 3), (P, Hkv, PAGE, D))
    _poison(k, v, table, seq_lens, poison)
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    return AttnCase(name, q, k, v, table, seq_lens, q_lens, scale)


def make_config(cfg, seed=0, poison=True):
    """Configurations 1..4 as (AttnCase, AcceptCase or None). Configuration 5
    is a job queue: use ``Config5Queue``."""
    lay = _rng(cfg, seed, 0)
    if cfg == 1:
        # 1 sequence of 300 tokens in 2 pages at random slots of a 16-page pool,
        # 8 q heads / 2 KV heads, head_dim 64, decode, accept over 32000 logits
        P, Hq, Hkv, D = 16, 8, 2, 64
        seq_lens = np.array([300], dtype=np.int32)
        q_lens = np.array([1], dtype=np.int32)
        table = lay.choice(P, 2, replace=False).astype(np.int32)[None, :]
        acc = _plant_drafts(_rng(cfg, seed, 4), _rng(cfg, seed, 5), q_lens, 32000)
    elif cfg == 2:
        # Llama3-8B-shaped decode: 64 sequences of U{512..1024} tokens in a
        # 256-page pool, tables are consecutive slices of one permutation
        P, Hq, Hkv, D = 256, 32, 8, 128
        seq_lens = lay.integers(512, 1025, 64).astype(np.int32)
        q_lens = np.ones(64, dtype=np.int32)
        perm = lay.permutation(P)
        table = np.full((64, 4), -1, dtype=np.int32)
        o = 0
        for b in range(64):
            n = _pages_for(seq_lens[b])
            table[b, :n] = perm[o:o + n]
            o += n
        acc = None
    elif cfg == 3:
        # speculative verify: 8 sequences x 8192 tokens fill the 256-page pool,
        # window of 6 rows (5 drafts + 1), accept over 128256 logits
        P, Hq, Hkv, D = 256, 32, 8, 128
        seq_lens = np.full(8, 8192, dtype=np.int32)
        q_lens = np.full(8, 6, dtype=np.int32)
        perm = lay.permutation(P)
        table = perm.reshape(8, 32).astype(np.int32)
        acc = _plant_drafts(_rng(cfg, seed, 4), _rng(cfg, seed, 5), q_lens, 128256)
    elif cfg == 4:
        # prefix dedup: 100 sequences share 16 physical pages (4096 tokens) and
        # own one private page of 1..256 tokens each
        P, Hq, Hkv, D = 256, 32, 8, 128
        perm = lay.permutation(P)
        shared = perm[:16]
        private = perm[16:116]
        r = lay.integers(1, 257, 100)
        seq_lens = (4096 + r).astype(np.int32)
        q_lens = np.ones(100, dtype=np.int32)
        table = np.empty((100, 17), dtype=np.int32)
        table[:, :16] = shared[None, :]
        table[:, 16] = private
        acc = None
    else:
        raise ValueError("make_config handles configurations 1..4; use Config5Queue for 5")
    q = _q_for(_rng(cfg, seed, 1), q_lens, Hq, D)
    k = _normal_bf16(_rng(cfg, seed, 2), (P, Hkv, PAGE, D))
    v = _normal_bf16(_rng(cfg, seed, 3), (P, Hkv, PAGE, D))
    _poison(k, v, table, seq_lens, poison)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    case = AttnCase(f"config{cfg}", q, k, v, table.astype(np.int32), seq_lens, q_lens, scale,
                    meta={"cfg": cfg, "seed": seed})
    return case, acc


def make_prefill_config(which, seed=0, poison=True):
    """Long-window (prefill) workloads on the shapes of configurations 3 and 4.

    * ``"full"``: the verify configuration's cache (8 sequences of 8192 tokens
      filling the 256-page pool, 32/8 heads, head_dim 128), every token a
      window row: q_len = seq_len = 8192, a whole-prompt prefill.
    * ``"dedup"``: the prefix-dedup layout of configuration 4 (100 sequences
      sharing 16 pages of prompt prefix, one private page of 1..256 tokens
      each); only the private tail is a window (q_len = tail length), the
      work that remains when the shared prefix is already cached.
    """
    if which == "full":
        case, _ = make_config(3, seed, poison)
        q_lens = case.seq_lens.copy()
    elif which == "dedup":
        case, _ = make_config(4, seed, poison)
        q_lens = (case.seq_lens - 4096).astype(np.int32)
    else:
        raise ValueError("which is 'full' or 'dedup'")
    Hq, D = case.num_q_heads, case.head_dim
    q = _q_for(_rng(200 + case.meta["cfg"], seed, 1), q_lens, Hq, D)
    return AttnCase(f"prefill-{which}", q, case.k_pool, case.v_pool, case.block_table, case.seq_lens,
                    q_lens.astype(np.int32), case.scale, meta={"cfg": case.meta["cfg"], "seed": seed,
                                                               "prefill": which})


# ---------------------------------------------------------------- layout transforms

def contiguous_twin(case):
    """Same sequences with each one's pages laid out consecutively, in order,
    in a fresh pool (the 'unpaged' layout: an identity-like table)."""
    B, W = case.block_table.shape
    pages = [_pages_for(s) for s in case.seq_lens]
    P2 = max(1, sum(pages))
    shape = (P2,) + case.k_pool.shape[1:]
    k = np.full(shape, BF16_QNAN, dtype=np.uint16)
    v = np.full(shape, BF16_QNAN, dtype=np.uint16)
    table = np.full((B, W), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        n = pages[b]
        src = case.block_table[b, :n]
        k[o:o + n] = case.k_pool[src]
        v[o:o + n] = case.v_pool[src]
        table[b, :n] = np.arange(o, o + n, dtype=np.int32)
        o += n
    return AttnCase(case.name + "-contig", case.q, k, v, table, case.seq_lens, case.q_lens,
                    case.scale, dict(case.meta))


def permute_pages(case, seed):
    """Move every physical page p to slot pi[p] and rewrite the tables."""
    rng = np.random.default_rng(np.random.SeedSequence([7, seed]))
    P = case.num_pages
    pi = rng.permutation(P).astype(np.int32)
    k = np.empty_like(case.k_pool)
    v = np.empty_like(case.v_pool)
    k[pi] = case.k_pool
    v[pi] = case.v_pool
    table = case.block_table.copy()
    valid = table >= 0
    table[valid] = pi[table[valid]]
    return AttnCase(case.name + "-perm", case.q, k, v, table, case.seq_lens, case.q_lens,
                    case.scale, dict(case.meta))


def duplicate_shared_pages(case):
    """Give every sequence private copies of all its pages (no page shared)."""
    B, W = case.block_table.shape
    pages = [_pages_for(s) for s in case.seq_lens]
    P2 = sum(pages)
    idx = np.concatenate([case.block_table[b, :pages[b]] for b in range(B)])
    k = case.k_pool[idx]
    v = case.v_pool[idx]
    table = np.full((B, W), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        table[b, :pages[b]] = np.arange(o, o + pages[b], dtype=np.int32)
        o += pages[b]
    assert o == P2
    return AttnCase(case.name + "-dup", case.q, k, v, table, case.seq_lens, case.q_lens,
                    case.scale, dict(case.meta))
