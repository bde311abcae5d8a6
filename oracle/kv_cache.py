"""Writing a verify window's K/V into the paged cache, and rolling back the
rejected part after the accept step (test oracle, plain Python loops).

Sources:

* ExLlamaV2 "Dynamic Generator" page, section "Continuous Batching": the cache
  is reached through per-sequence block tables of fixed 256-token pages; a
  sequence grows into pages handed to it, changing a batch only rewrites block
  indices, and pages freed by a finished job leave holes that later jobs fill
  (indices need not be contiguous).
* Hugging Face "Assisted Generation" page, section "Assisted Generation loop",
  step 4: candidates after the first mismatch are discarded, so their cache
  entries go too; the kept tokens are the matching prefix plus the window's
  first token (the accepted count of the accept step).

Readings taken (the pages fix no allocator):

* free pages form a stack ``free_pages[0:count]``; an append pops pages from
  the top, sequences in index order and each sequence's new pages in table
  order; a rollback pushes released pages on top in the same order;
* ``seq_lens`` counts cached tokens; an append writes window token ``i`` of
  sequence ``b`` at position ``seq_len + i`` (slot ``pos % 256`` of page
  ``table[b][pos // 256]``) and adds ``q_len``; a rollback sets the length to
  ``seq_len - q_len + accepted`` and releases every page past the new length;
* a page that receives appended tokens belongs to that sequence alone (pages
  shared for dedup are full prefix pages);
* any broken contract (lengths, table width, too few free pages) leaves every
  buffer unchanged; here it raises ``ValueError``.

Layouts: pools uint16 bf16 bits [P, Hkv, 256, D]; new rows uint16
[sum(q_lens), Hkv, D] packed by sequence; block_table int32 [B, W] with -1 for
no page; free_pages int32 [P].
"""

import numpy as np

PAGE = 256


def _pages(n_tokens):
    return -(-int(n_tokens) // PAGE)


def append(k_pool, v_pool, block_table, seq_lens, q_lens, k_new, v_new, free_pages, free_count):
    """Returns new (k_pool, v_pool, block_table, seq_lens, free_pages,
    free_count); the inputs are not modified."""
    k_pool, v_pool = k_pool.copy(), v_pool.copy()
    table = np.array(block_table, dtype=np.int32, copy=True)
    lens = np.array(seq_lens, dtype=np.int64, copy=True)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    free = np.array(free_pages, dtype=np.int32, copy=True)
    B, W = table.shape
    if k_new.shape[0] != int(q_lens.sum()) or v_new.shape != k_new.shape:
        raise ValueError("new rows must be sum(q_lens)")
    need = 0
    for b in range(B):
        if lens[b] < 0 or q_lens[b] < 0 or lens[b] + q_lens[b] > W * PAGE:
            raise ValueError(f"sequence {b}: lengths out of range")
        need += _pages(lens[b] + q_lens[b]) - _pages(lens[b])
    if need > free_count:
        raise ValueError("not enough free pages")
    top = int(free_count)
    row = 0
    for b in range(B):
        L, n = int(lens[b]), int(q_lens[b])
        for j in range(_pages(L), _pages(L + n)):   # pages the window grows into
            top -= 1
            table[b, j] = free[top]
        for i in range(n):
            pos = L + i
            page, slot = int(table[b, pos // PAGE]), pos % PAGE
            k_pool[page, :, slot, :] = k_new[row + i]
            v_pool[page, :, slot, :] = v_new[row + i]
        row += n
        lens[b] = L + n
    return k_pool, v_pool, table, lens.astype(np.int32), free, top


def rollback(block_table, seq_lens, q_lens, accepted, free_pages, free_count):
    """Keep the first ``accepted`` window tokens of each sequence. Returns new
    (block_table, seq_lens, free_pages, free_count)."""
    table = np.array(block_table, dtype=np.int32, copy=True)
    lens = np.array(seq_lens, dtype=np.int64, copy=True)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    accepted = np.asarray(accepted, dtype=np.int64)
    free = np.array(free_pages, dtype=np.int32, copy=True)
    B, W = table.shape
    released = 0
    for b in range(B):
        S, n, a = int(lens[b]), int(q_lens[b]), int(accepted[b])
        if not (0 <= a <= n <= S) or _pages(S) > W:
            raise ValueError(f"sequence {b}: lengths out of range")
        released += _pages(S) - _pages(S - n + a)
    if free_count + released > free.shape[0]:
        raise ValueError("free list would overflow")
    top = int(free_count)
    for b in range(B):
        S, n, a = int(lens[b]), int(q_lens[b]), int(accepted[b])
        new_len = S - n + a
        for j in range(_pages(new_len), _pages(S)):   # pages wholly past the kept tokens
            free[top] = table[b, j]
            top += 1
            table[b, j] = -1
        lens[b] = new_len
    return table, lens.astype(np.int32), free, top
