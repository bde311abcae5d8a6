"""Pins of the Q8 cache oracle (oracle/q8_cache.py) against what the
definition fixes: the round-trip error bound, exact codes for exact
multiples, the largest value on +-127, ties to even, sign symmetry and
power-of-two scaling, zero and non-finite vectors, and a per-element scalar
re-derivation on small inputs."""

import numpy as np

from oracle import q8_cache as q8
from workloads import normal_bf16


def f32_to_bf16_exact(x):
    """bf16 bits of values that are exactly representable (test inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "not exact in bf16"
    return (u >> 16).astype(np.uint16)


def widen(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_round_trip_error_is_bounded():
    rng = np.random.default_rng(1)
    x = normal_bf16(rng, (200, 128))
    c, s = q8.encode(x)
    d = q8.decode(c, s)
    xf = widen(x)
    # half a quantization step (the binary32 quotient's own rounding adds at
    # most 127 * 2^-24 of a step); the decoded value is the exact product
    bound = s[:, None].astype(np.float64) * (0.5 + 2.0 ** -16)
    assert np.all(np.abs(d - xf) <= bound)
    assert np.all(np.abs(c) <= 127)


def test_largest_value_maps_to_127():
    rng = np.random.default_rng(2)
    x = normal_bf16(rng, (50, 64))
    c, _ = q8.encode(x)
    xf = widen(x)
    i = np.argmax(np.abs(xf), axis=1)
    assert np.all(np.abs(c[np.arange(50), i]) == 127)
    assert np.all(np.sign(c[np.arange(50), i]) == np.sign(xf[np.arange(50), i]))


def test_exact_multiples_encode_and_decode_exactly():
    k = np.arange(-127, 128, dtype=np.float32)
    x = f32_to_bf16_exact(k * np.float32(2.0 ** -4))[None, :]
    c, s = q8.encode(x)
    assert s[0] == np.float32(2.0 ** -4)
    assert np.array_equal(c[0], k.astype(np.int8))
    assert np.array_equal(q8.decode(c, s), widen(x))


def test_ties_go_to_even():
    # scale 2^-4 (max 127 * 2^-4): 2.5, 3.5, -2.5 steps round to 2, 4, -2
    vals = np.zeros(16, np.float32)
    vals[0] = 127 * 2.0 ** -4
    vals[1], vals[2], vals[3] = 2.5 * 2.0 ** -4, 3.5 * 2.0 ** -4, -2.5 * 2.0 ** -4
    c, s = q8.encode(f32_to_bf16_exact(vals)[None, :])
    assert s[0] == np.float32(2.0 ** -4)
    assert list(c[0, :4]) == [127, 2, 4, -2]


def test_sign_symmetry_and_power_of_two_scaling():
    rng = np.random.default_rng(3)
    x = normal_bf16(rng, (40, 128))
    c, s = q8.encode(x)
    cn, sn = q8.encode(x ^ np.uint16(0x8000))          # -x
    assert np.array_equal(cn, -c) and np.array_equal(sn, s)
    x2 = f32_to_bf16_exact(widen(x).astype(np.float32) * np.float32(2.0))
    c2, s2 = q8.encode(x2)
    assert np.array_equal(c2, c) and np.array_equal(s2, s * np.float32(2.0))


def test_zero_and_non_finite_vectors():
    z = np.zeros((2, 64), np.uint16)
    z[1, 3] = 0x8000                                     # -0.0
    c, s = q8.encode(z)
    assert np.all(c == 0) and np.all(s == 0)
    assert np.all(q8.decode(c, s) == 0)
    bad = np.full((3, 64), 0x3F80, np.uint16)            # 1.0
    bad[0, 5] = 0x7FC0                                   # NaN
    bad[1, 9] = 0x7F80                                   # +inf
    c, s = q8.encode(bad)
    assert np.isnan(s[0]) and np.isnan(s[1]) and s[2] == np.float32(1.0 / 127)
    assert np.all(c[:2] == 0) and np.all(c[2] == 127)
    d = q8.decode(c, s)
    assert np.all(np.isnan(d[:2]))
    # 127 times binary32(1/127) = 0.0078740157186985015869140625, exactly
    assert np.all(d[2] == 0.9999999962747097015380859375)


def test_scalar_rederivation_on_small_vectors():
    """Each element taken alone, with numpy float32 scalars: the scale from the
    largest magnitude, the quotient, round half to even by hand; the decoded
    value is the code times the scale in Python's (binary64) arithmetic."""
    rng = np.random.default_rng(4)
    x = normal_bf16(rng, (6, 16))
    c, s = q8.encode(x)
    d = q8.decode(c, s)
    for r in range(6):
        vals = [np.float32(v) for v in widen(x[r])]
        amax = np.float32(0)
        for v in vals:
            amax = max(amax, np.float32(abs(v)))
        scale = np.float32(amax / np.float32(127))
        assert scale == s[r]
        for j, v in enumerate(vals):
            t = np.float32(v / scale)
            lo = np.floor(float(t))
            frac = float(t) - lo
            code = lo + 1 if frac > 0.5 or (frac == 0.5 and lo % 2 == 1) else lo
            assert int(code) == int(c[r, j])
            assert d[r, j] == int(code) * float(scale)


def test_decoded_values_worked_by_hand():
    """Products worked out by hand: scale 1/8 on 127, -1 and 0; binary32(0.1)
    = 0.100000001490116119384765625 on 100 and -128; the subnormal-range
    scale 2^-140 on -128 (a binary64 normal number)."""
    d = q8.decode(np.array([[127, -1, 0]], np.int8), np.array([0.125], np.float32))
    assert list(d[0]) == [15.875, -0.125, 0.0]
    d = q8.decode(np.array([[100, -128]], np.int8), np.array([0.1], np.float32))
    assert list(d[0]) == [10.0000001490116119384765625, -12.80000019073486328125]
    d = q8.decode(np.array([[-128]], np.int8), np.array([2.0 ** -140], np.float32))
    assert d[0, 0] == -(2.0 ** -133)
