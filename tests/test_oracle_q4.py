"""Pins of the Q4 cache oracle (oracle/q4_cache.py) against what the
definition fixes: the round-trip error bound, exact codes for exact multiples,
the largest value on +-7, ties to even, the nibble order of the packing, sign
symmetry and power-of-two scaling, zero and non-finite vectors, and a
per-element scalar re-derivation (codes, packed bytes, decoded bits) on small
inputs."""

import numpy as np

from oracle import q4_cache as q4
from workloads import normal_bf16


def f32_to_bf16_exact(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "not exact in bf16"
    return (u >> 16).astype(np.uint16)


def widen(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_round_trip_error_is_bounded():
    rng = np.random.default_rng(11)
    x = normal_bf16(rng, (200, 128))
    p, s = q4.encode(x)
    c = q4.unpack(p)
    d = q4.decode(p, s)
    # half a quantization step (plus the binary32 quotient's rounding); the
    # decoded value is the exact product
    bound = s[:, None].astype(np.float64) * (0.5 + 2.0 ** -20)
    assert np.all(np.abs(d - widen(x)) <= bound)
    assert np.all(np.abs(c) <= 7)
    assert p.shape == (200, 64) and p.dtype == np.uint8


def test_largest_value_maps_to_7():
    rng = np.random.default_rng(12)
    x = normal_bf16(rng, (50, 64))
    c, _ = q4.codes_of(x)
    xf = widen(x)
    i = np.argmax(np.abs(xf), axis=1)
    assert np.all(np.abs(c[np.arange(50), i]) == 7)
    assert np.all(np.sign(c[np.arange(50), i]) == np.sign(xf[np.arange(50), i]))


def test_exact_multiples_and_the_nibble_order():
    k = np.array([-7, -6, -5, -4, -3, -2, -1, 0, 1, 2, 3, 4, 5, 6, 7, 7], np.float32)
    x = f32_to_bf16_exact(k * np.float32(0.5))[None, :]
    p, s = q4.encode(x)
    assert s[0] == np.float32(0.5)
    # byte i = (code[2i] + 8) | (code[2i + 1] + 8) << 4
    assert list(p[0]) == [(1 | 2 << 4), (3 | 4 << 4), (5 | 6 << 4), (7 | 8 << 4),
                          (9 | 10 << 4), (11 | 12 << 4), (13 | 14 << 4), (15 | 15 << 4)]
    assert np.array_equal(q4.unpack(p)[0], k.astype(np.int8))
    assert np.array_equal(q4.decode(p, s), widen(x))


def test_ties_go_to_even():
    # scale 1 (max 7): 2.5, 3.5, -2.5, 0.5, -1.5 round to 2, 4, -2, 0, -2
    vals = np.zeros(16, np.float32)
    vals[:6] = [7.0, 2.5, 3.5, -2.5, 0.5, -1.5]
    c, s = q4.codes_of(f32_to_bf16_exact(vals)[None, :])
    assert s[0] == np.float32(1.0)
    assert list(c[0, :6]) == [7, 2, 4, -2, 0, -2]


def test_sign_symmetry_and_power_of_two_scaling():
    rng = np.random.default_rng(13)
    x = normal_bf16(rng, (40, 128))
    c, s = q4.codes_of(x)
    cn, sn = q4.codes_of(x ^ np.uint16(0x8000))
    assert np.array_equal(cn, -c) and np.array_equal(sn, s)
    x2 = f32_to_bf16_exact(widen(x).astype(np.float32) * np.float32(4.0))
    c2, s2 = q4.codes_of(x2)
    assert np.array_equal(c2, c) and np.array_equal(s2, s * np.float32(4.0))


def test_zero_and_non_finite_vectors():
    z = np.zeros((2, 64), np.uint16)
    z[1, 3] = 0x8000
    p, s = q4.encode(z)
    assert np.all(p == 0x88) and np.all(s == 0)
    assert np.all(q4.decode(p, s) == 0)
    bad = np.full((3, 64), 0x3F80, np.uint16)
    bad[0, 5] = 0x7FC0
    bad[1, 9] = 0xFF80                                   # -inf
    p, s = q4.encode(bad)
    assert np.isnan(s[0]) and np.isnan(s[1]) and s[2] == np.float32(1.0 / 7)
    assert np.all(p[:2] == 0x88) and np.all(p[2] == 0xFF)
    d = q4.decode(p, s)
    assert np.all(np.isnan(d[:2]))
    # 7 times binary32(1/7) = 0.14285714924335479736328125, exactly
    assert np.all(d[2] == 1.00000004470348358154296875)


def test_scalar_rederivation_on_small_vectors():
    """Element by element with numpy float32 scalars: scale, quotient, round
    half to even by hand, the nibble pair of each byte; the decoded value is
    the code times the scale in Python's (binary64) arithmetic."""
    rng = np.random.default_rng(14)
    x = normal_bf16(rng, (6, 16))
    p, s = q4.encode(x)
    d = q4.decode(p, s)
    for r in range(6):
        vals = [np.float32(v) for v in widen(x[r])]
        amax = np.float32(0)
        for v in vals:
            amax = max(amax, np.float32(abs(v)))
        scale = np.float32(amax / np.float32(7))
        assert scale == s[r]
        codes = []
        for j, v in enumerate(vals):
            t = np.float32(v / scale)
            lo = np.floor(float(t))
            frac = float(t) - lo
            code = lo + 1 if frac > 0.5 or (frac == 0.5 and lo % 2 == 1) else lo
            code = int(max(-7, min(7, code)))
            codes.append(code)
            assert d[r, j] == code * float(scale)
        for i in range(8):
            assert int(p[r, i]) == (codes[2 * i] + 8) + 16 * (codes[2 * i + 1] + 8)


def test_every_byte_decodes_to_its_nibble_pair():
    """All 256 bytes at scale 1: byte b holds codes (b & 15) - 8 (even dim)
    and (b >> 4) - 8 (odd dim), decoded exactly; and products worked out by
    hand at binary32(0.3) = 0.300000011920928955078125 and at 2^-130."""
    b = np.arange(256, dtype=np.uint8).reshape(256, 1)
    d = q4.decode(b, np.ones(256, np.float32))
    for v in range(256):
        assert d[v, 0] == (v & 15) - 8 and d[v, 1] == (v >> 4) - 8
    d = q4.decode(np.array([[0x0F, 0xF0]], np.uint8), np.array([0.3], np.float32))
    # bytes 0x0F, 0xF0: codes (7, -8), (-8, 7)
    assert list(d[0]) == [2.100000083446502685546875, -2.4000000953674316406250,
                          -2.4000000953674316406250, 2.100000083446502685546875]
    d = q4.decode(np.array([[0x00]], np.uint8), np.array([2.0 ** -130], np.float32))
    assert list(d[0]) == [-(2.0 ** -127), -(2.0 ** -127)]
