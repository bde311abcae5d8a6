"""Quantized (Q8) paged K/V cache, the plain definition (test oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: ExLlamaV2 "Dynamic Generator" page, section "Usage" (preparing the
model and the generator): the generator takes a 4-bit (Q4) cache mode in place
of the plain cache, an FP8 cache is left out because Q4 beats it, and an 8-bit
(Q8) mode is announced as about as compact as FP8 but more accurate. The page
gives no format. Readings taken (the plainest the page supports):

* more accurate than FP8 at about its size: 8-bit integer codes with a
  per-vector scale (8 significant bits against FP8's 3 or 4), one vector being
  the D values of one token in one KV head of one page; the scale is fp32, so
  a token costs D + 4 bytes per KV head (132 against 256 for bf16 at D 128);
* symmetric quantization: ``scale = max|x| / 127``, ``code = round(x / scale)``
  to nearest with ties to even, codes in [-127, 127]; a zero vector has scale
  0 and codes 0; a vector holding a non-finite value gets scale NaN and codes
  0 (its decoded values are NaN, like the unused slots of a bf16 pool);
* all of it in IEEE binary32 (the inputs are bf16, exact in binary32);
* decoding: ``code * scale``, the exact real product (exact in float64: 8
  bits times 24). Attention over a Q8 cache is attention over the decoded
  pools, with every other definition unchanged.

Layouts: codes int8 [..., D] and scales float32 [...] for bf16 bits
uint16 [..., D] (pools: [P, Hkv, 256, D] and [P, Hkv, 256]); decoded values
float64 [..., D].
"""

import numpy as np

QMAX = np.float32(127.0)


def _widen(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def encode(bits):
    """bf16 vectors (last axis) -> (int8 codes, float32 scales)."""
    x = _widen(bits)
    finite = np.all(np.isfinite(x), axis=-1)
    amax = np.max(np.abs(np.where(np.isfinite(x), x, np.float32(0))), axis=-1).astype(np.float32)
    scale = (amax / QMAX).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1)).astype(np.float32)
    with np.errstate(invalid="ignore"):
        q = np.rint(np.where(np.isfinite(x), x, np.float32(0)) / safe[..., None]).astype(np.float32)
    codes = np.clip(q, -127, 127).astype(np.int8)
    codes = np.where((scale > 0)[..., None] & finite[..., None], codes, np.int8(0)).astype(np.int8)
    scale = np.where(finite, scale, np.float32(np.nan)).astype(np.float32)
    return codes, scale


def decode(codes, scales):
    """(int8 codes, float32 scales) -> float64 values code * scale (NaN where
    the scale is NaN)."""
    c = np.asarray(codes, dtype=np.int8).astype(np.float64)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None]
    with np.errstate(invalid="ignore"):
        return c * s
