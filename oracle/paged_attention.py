"""Paged K/V attention, the plain definition in float64 (test oracle).

Sources and readings:

* ExLlamaV2 "Dynamic Generator" page, section "Continuous Batching": the K/V
  cache is addressed through a block table of fixed 256-token pages; adding or
  removing a sequence only rewrites block indices, and the indices need not be
  contiguous (freed pages leave holes that new jobs fill).
* Same page, section "Deduplication": several sequences may index the same
  page (a shared prefix is stored once).
* Hugging Face "Assisted Generation" page, section "How Assisted Generation
  works": one forward pass over a token window yields logits at every window
  position, so attention serves q_len = k + 1 rows per sequence.

The pages print no attention equation. Readings taken (each is the plainest one
the rest supports):

* scaled dot-product softmax attention, ``softmax(scale * q . k) . v``;
* grouped-query heads: q head ``h`` reads KV head ``h // (Hq // Hkv)``;
* ``seq_len`` counts the verify window (its K/V are already in the pages);
  window row ``i`` of ``q_len`` sees keys ``0 .. seq_len - q_len + i``;
* slots of the last page past ``seq_len`` and table entries past
  ``ceil(seq_len / 256)`` are never read;
* inputs are bf16 bit patterns; they are widened exactly to float64.

Layouts: q uint16 [total_q, Hq, D] packed by sequence then window row; pools
uint16 [P, Hkv, 256, D]; block_table int32 [B, W]; out float64 [total_q, Hq, D].
"""

import numpy as np

PAGE = 256


def decode_bf16(bits):
    """Widen bf16 bit patterns exactly to float64: the 16 bits are the top
    half of an IEEE binary32 value."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def gather_sequence(pool_bits, table_row, seq_len):
    """Contiguous [Hkv, seq_len, D] bits of one sequence: its pages in table
    order, concatenated along the token axis, cut to seq_len tokens."""
    P = pool_bits.shape[0]
    n_pages = -(-int(seq_len) // PAGE)
    pages = np.asarray(table_row[:n_pages], dtype=np.int64)
    if np.any(pages < 0) or np.any(pages >= P):
        raise ValueError(f"block table entry outside [0, {P}): {pages}")
    tiles = pool_bits[pages]                       # [n_pages, Hkv, 256, D]
    hkv, d = tiles.shape[1], tiles.shape[3]
    seq = tiles.transpose(1, 0, 2, 3).reshape(hkv, n_pages * PAGE, d)
    return seq[:, :seq_len, :]


def attention_rows(q_rows, K, V, q_len, seq_len, scale):
    """Exact attention of one sequence's window.

    q_rows float64 [q_len, Hq, D]; K, V float64 [Hkv, seq_len, D].
    Returns float64 [q_len, Hq, D].
    """
    q_len, Hq, D = q_rows.shape
    Hkv = K.shape[0]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    out = np.empty((q_len, Hq, D), dtype=np.float64)
    for i in range(q_len):
        last = seq_len - q_len + i            # newest key this window row may see
        if last < 0:
            raise ValueError("q_len exceeds seq_len")
        for h in range(Hq):
            g = h // group
            s = scale * (K[g, :last + 1] @ q_rows[i, h])
            s = s - s.max()
            p = np.exp(s)
            p /= p.sum()
            out[i, h] = p @ V[g, :last + 1]
    return out


def _attention(q_bits, k_pool, v_pool, block_table, seq_lens, q_lens, scale, widen):
    q = decode_bf16(q_bits)
    total_q, Hq, D = q.shape
    out = np.zeros((total_q, Hq, D), dtype=np.float64)
    scale = float(scale)
    r0 = 0
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        ql = int(q_lens[b])
        if ql == 0:
            continue
        K = widen(gather_sequence(k_pool, block_table[b], L))
        V = widen(gather_sequence(v_pool, block_table[b], L))
        out[r0:r0 + ql] = attention_rows(q[r0:r0 + ql], K, V, ql, L, scale)
        r0 += ql
    if r0 != total_q:
        raise ValueError(f"sum(q_lens) = {r0} but q has {total_q} rows")
    return out


def attention(q_bits, k_pool_bits, v_pool_bits, block_table, seq_lens, q_lens, scale):
    """Paged attention over a batch: float64 [total_q, Hq, D]."""
    return _attention(q_bits, k_pool_bits, v_pool_bits, block_table, seq_lens, q_lens, scale, decode_bf16)


def attention_decoded(q_bits, k_pool_vals, v_pool_vals, block_table, seq_lens, q_lens, scale):
    """The same over pools already holding the cached values as float64
    [P, Hkv, 256, D] (a quantized cache's decoded pools)."""
    return _attention(q_bits, k_pool_vals, v_pool_vals, block_table, seq_lens, q_lens, scale,
                      lambda x: np.asarray(x, dtype=np.float64))
