"""Helpers shared by the tests: turn golden JSON cases into input arrays."""

import json
import os

import numpy as np

from workloads import f32_to_bf16_bits, AttnCase

PAGE = 256
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _pool(c, which):
    P, Hkv, D = c["num_pages"], c["Hkv"], c["D"]
    fill = c[which + "_fill"]
    arr = np.full((P, Hkv, PAGE, D), np.nan if fill == "nan" else float(fill), dtype=np.float32)
    for page, head, s0, s1, d, val in c[which + "_entries"]:
        arr[page, head, s0:s1, d] = val
    return f32_to_bf16_bits(arr)


def golden_attention_case(c):
    q = f32_to_bf16_bits(np.array(c["q"], dtype=np.float32))
    return AttnCase(c["name"], q, _pool(c, "k"), _pool(c, "v"),
                    np.array(c["block_table"], dtype=np.int32),
                    np.array(c["seq_lens"], dtype=np.int32),
                    np.array(c["q_lens"], dtype=np.int32),
                    float(np.float32(c["scale"])))
