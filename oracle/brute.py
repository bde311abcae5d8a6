"""Brute force for tiny inputs: pure-Python loops, one token and one element
at a time, with its own bf16 decoding and its own page lookup. It exists to pin
``paged_attention`` and ``accept``; it shares nothing with them.

Token ``t`` of sequence ``b`` is slot ``t % 256`` of page
``block_table[b][t // 256]`` (ExLlamaV2 "Dynamic Generator" page, section
"Continuous Batching": pages of 256 tokens reached through the block table).
"""

import math
import struct

PAGE = 256


def _bf16(bits):
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def attention_brute(q_bits, k_pool_bits, v_pool_bits, block_table, seq_lens, q_lens, scale):
    """Nested lists [total_q][Hq][D] of Python floats."""
    total_q, Hq, D = q_bits.shape
    Hkv = k_pool_bits.shape[1]
    group = Hq // Hkv
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(total_q)]
    row = 0
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        ql = int(q_lens[b])
        for i in range(ql):
            visible = L - ql + i + 1
            for h in range(Hq):
                g = h // group
                qv = [_bf16(q_bits[row, h, d]) for d in range(D)]
                scores = []
                for t in range(visible):
                    page = int(block_table[b][t // PAGE])
                    slot = t % PAGE
                    kv = [_bf16(k_pool_bits[page, g, slot, d]) for d in range(D)]
                    scores.append(float(scale) * math.fsum(a * c for a, c in zip(qv, kv)))
                top = max(scores)
                w = [math.exp(s - top) for s in scores]
                z = math.fsum(w)
                for d in range(D):
                    terms = []
                    for t in range(visible):
                        page = int(block_table[b][t // PAGE])
                        terms.append(w[t] * _bf16(v_pool_bits[page, g, t % PAGE, d]))
                    out[row][h][d] = math.fsum(terms) / z
            row += 1
    return out


def argmax_brute(row):
    """First NaN if there is one, else the lowest index of the maximum."""
    best_i, best = 0, None
    for i, x in enumerate(row):
        x = float(x)
        if math.isnan(x):
            return i
        if best is None or x > best:
            best_i, best = i, x
    return best_i


def accept_brute(pred_rows, drafts):
    """Accepted count by trying every prefix length from the longest down:
    the longest k with drafts[:k] == preds[:k], plus the kept base token."""
    n = len(drafts)
    for k in range(n, -1, -1):
        if all(pred_rows[i] == drafts[i] for i in range(k)):
            return k + 1, pred_rows[k]
    raise AssertionError("unreachable")
