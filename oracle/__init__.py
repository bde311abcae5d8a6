"""CPU oracle for paged K/V attention and the greedy speculative accept step.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU library
never calls it, and it shares no code with the GPU library: it reads the data
layout from the C header's documentation only and decodes every input itself.

What it computes is the plain definition, in float64:

* ``paged_attention.attention`` -- materialise each sequence's contiguous K/V
  from its block table, then exact softmax attention with the verify window
  causal inside the window (``paged_attention`` module docstring lists the
  readings of the pages it follows).
* ``greedy_accept.argmax_rows`` / ``.accept`` / ``.window_next`` -- the
  vocab-wide argmax, the left-to-right draft comparison with one correction
  token, and the +2 / -1 draft-window rule.
* ``kv_cache.append`` / ``.rollback`` -- writing a verify window's K/V into
  the pages (popping new pages from a free stack) and, after the accept,
  keeping the accepted prefix and releasing the pages past it.
* ``page_pool.PagePool`` -- the page allocator: reference counts, prefix
  reuse at admission, prompt caching with least-recently-released eviction,
  and defragmentation; ``page_pool.copy_pages`` / ``.remap_table`` for the
  data movement a defragmentation plans.
* ``q8_cache.encode`` / ``.decode`` -- the Q8 cache: 8-bit codes with one
  fp32 scale per token vector, and the values they decode to, code x scale
  exactly (attention over a Q8 cache is ``attention_decoded`` over the
  decoded pools).
* ``q4_cache.encode`` / ``.decode`` -- the Q4 cache: the same scheme at 4
  bits (codes in [-7, 7], two nibbles per byte).
* ``brute`` -- an independent pure-Python loop version of the attention, per
  token and per element, used to pin ``paged_attention`` on tiny inputs.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
brute force, closed forms, invariants and hand-worked fixtures under
``tests/golden/``. Absolute attention values at the full configuration sizes
have no printed reference on the pages; they are pinned only through those
checks.
"""

from .paged_attention import decode_bf16, gather_sequence, attention, attention_decoded, attention_rows
from .greedy_accept import argmax_rows, accept, window_next
from . import kv_cache
from . import page_pool
from . import q8_cache
from . import q4_cache

__all__ = ["decode_bf16", "gather_sequence", "attention", "attention_rows",
           "argmax_rows", "accept", "window_next", "kv_cache", "page_pool", "q8_cache", "q4_cache"]
