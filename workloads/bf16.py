"""bfloat16 bit-pattern encoding for synthetic inputs.

Inputs are drawn as float32 and rounded to bf16 with round-to-nearest-even,
then handed to both sides as raw uint16 bit patterns, so the rounding never
affects parity: the oracle and the kernels decode the very same bits.
"""

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)


_CHUNK = 1 << 20


def _round_chunk(src, dst):
    u = src.view(np.uint32).copy()
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    dst[:] = u
    nan = np.isnan(src)
    if nan.any():
        dst[nan] = BF16_QNAN


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Adding 0x7FFF plus the lowest kept bit and truncating rounds to nearest
    with ties to even. NaN inputs map to the canonical quiet NaN 0x7FC0.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    fi, fo = x.reshape(-1), out.reshape(-1)
    for s in range(0, fi.size, _CHUNK):
        _round_chunk(fi[s:s + _CHUNK], fo[s:s + _CHUNK])
    return out


def normal_bf16(rng, shape):
    """N(0, 1) float32 draws rounded to bf16 bits, drawn in 2^20-element
    chunks (row-major order) so the float32 copy never exists whole."""
    out = np.empty(shape, dtype=np.uint16)
    fo = out.reshape(-1)
    for s in range(0, fo.size, _CHUNK):
        n = min(_CHUNK, fo.size - s)
        _round_chunk(rng.standard_normal(n, dtype=np.float32), fo[s:s + n])
    return out


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to float32 (for generators only)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
