"""Seeded synthetic inputs for the paged K/V attention path and the greedy
speculative accept step.

This package only draws numbers and lays them out (bf16 bit patterns, block
tables, page pools, logits, draft ids). It computes no attention, no softmax
and no argmax: both the CPU oracle and the GPU path consume what it produces,
and neither imports the other.

Layouts (the ones the C ABI documents):
  q        bf16 bits uint16 [total_q, Hq, D], packed by sequence then window row
  k/v pool bf16 bits uint16 [P, Hkv, 256, D]
  block_table int32 [B, max_pages_per_seq] (entries past a sequence's pages = -1)
  seq_lens, q_lens int32 [B]; seq_len counts the verify window
  logits   float32 [sum(n_draft + 1), V], same row order as q
  draft_ids int32 packed [sum(n_draft)]
"""

from .bf16 import f32_to_bf16_bits, bf16_bits_to_f32, normal_bf16, BF16_QNAN
from .configs import (
    PAGE,
    AttnCase,
    AcceptCase,
    make_config,
    make_prefill_config,
    make_tiny_case,
    make_accept_case,
    kv_logical_bytes,
    contiguous_twin,
    permute_pages,
    duplicate_shared_pages,
)
from .churn import Config5Queue

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "BF16_QNAN", "PAGE", "AttnCase", "AcceptCase",
    "make_config", "make_prefill_config", "make_tiny_case", "make_accept_case", "kv_logical_bytes",
    "contiguous_twin", "permute_pages", "duplicate_shared_pages", "Config5Queue",
]
