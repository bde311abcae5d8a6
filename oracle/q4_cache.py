"""Quantized (Q4) paged K/V cache, the plain definition (test oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: ExLlamaV2 "Dynamic Generator" page, section "Usage" (preparing the
model and the generator): the generator's quantized cache mode is a 4-bit
(Q4) cache, preferred there over an FP8 cache; the page gives no format.
Reading taken: the Q8 scheme of ``q8_cache`` at 4 bits, the plainest one the
page supports:

* per vector of D values (one token, one KV head, one page slot) one fp32
  ``scale = max|x| / 7``; ``code = round(x / scale)`` to nearest with ties to
  even, codes in [-7, 7]; a zero vector has scale 0 and codes 0; a vector
  holding a non-finite value gets scale NaN and codes 0;
* all in IEEE binary32 (the bf16 inputs are exact there);
* storage: the nibble ``code + 8`` (1 .. 15; 8 for a zero code), two per
  byte, dim 2i in the low nibble of byte i and dim 2i + 1 in the high one;
* decoding: ``code * scale`` exactly, as for Q8. Attention over a Q4 cache
  is attention over the decoded pools.

Layouts: packed uint8 [..., D / 2] and scales float32 [...] for bf16 bits
uint16 [..., D] (pools: [P, Hkv, 256, D / 2] and [P, Hkv, 256]); decoded
values float64 [..., D].
"""

import numpy as np

from .q8_cache import _widen

QMAX = np.float32(7.0)


def codes_of(bits):
    """bf16 vectors (last axis) -> (int8 codes in [-7, 7], float32 scales)."""
    x = _widen(bits)
    finite = np.all(np.isfinite(x), axis=-1)
    amax = np.max(np.abs(np.where(np.isfinite(x), x, np.float32(0))), axis=-1).astype(np.float32)
    scale = (amax / QMAX).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1)).astype(np.float32)
    with np.errstate(invalid="ignore"):
        q = np.rint(np.where(np.isfinite(x), x, np.float32(0)) / safe[..., None]).astype(np.float32)
    codes = np.clip(q, -7, 7).astype(np.int8)
    codes = np.where((scale > 0)[..., None] & finite[..., None], codes, np.int8(0)).astype(np.int8)
    scale = np.where(finite, scale, np.float32(np.nan)).astype(np.float32)
    return codes, scale


def pack(codes):
    """int8 codes [..., D] -> uint8 [..., D / 2]: nibble code + 8, even dims low."""
    n = (np.asarray(codes, np.int16) + 8).astype(np.uint8)
    return (n[..., 0::2] | (n[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack(packed):
    """uint8 [..., D / 2] -> int8 codes [..., D]."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.int8)
    out[..., 0::2] = (p & np.uint8(15)).astype(np.int8) - 8
    out[..., 1::2] = (p >> np.uint8(4)).astype(np.int8) - 8
    return out


def encode(bits):
    """bf16 vectors (last axis) -> (packed uint8 codes, float32 scales)."""
    codes, scale = codes_of(bits)
    return pack(codes), scale


def decode(packed, scales):
    """(packed uint8 codes, float32 scales) -> float64 values code * scale
    (NaN where the scale is NaN)."""
    c = unpack(packed).astype(np.float64)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None]
    with np.errstate(invalid="ignore"):
        return c * s
