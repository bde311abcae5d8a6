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
    d = widen(q8.decode(c, s))
    xf = widen(x)
    # half a quantization step, plus the bf16 rounding of the product
    bound = s[:, None] / 2 + np.abs(c * s[:, None].astype(np.float64)) * 2.0 ** -8
    assert np.all(np.abs(d - xf) <= bound + 1e-12)
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
    assert np.array_equal(q8.decode(c, s), x)


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
    assert np.all(widen(q8.decode(c, s)) == 0)
    bad = np.full((3, 64), 0x3F80, np.uint16)            # 1.0
    bad[0, 5] = 0x7FC0                                   # NaN
    bad[1, 9] = 0x7F80                                   # +inf
    c, s = q8.encode(bad)
    assert np.isnan(s[0]) and np.isnan(s[1]) and s[2] == np.float32(1.0 / 127)
    assert np.all(c[:2] == 0) and np.all(c[2] == 127)
    d = widen(q8.decode(c, s))
    assert np.all(np.isnan(d[:2])) and np.all(d[2] == 1.0)


def test_scalar_rederivation_on_small_vectors():
    """Each element taken alone, with numpy float32 scalars: the scale from the
    largest magnitude, the quotient, round half to even by hand, the product
    and its bf16 rounding by hand (truncate, then round on the dropped half)."""
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
            prod = np.float32(np.float32(code) * scale)
            u = int(np.array([prod], np.float32).view(np.uint32)[0])
            hi, low = u >> 16, u & 0xFFFF
            if low > 0x8000 or (low == 0x8000 and hi & 1):
                hi += 1
            assert hi == int(d[r, j])


def test_every_code_decodes_to_the_rounded_product():
    """All 256 codes at scales 1, 1/127, an odd value and a subnormal: the
    decoded bf16 is the float32 product rounded to nearest even, by hand."""
    c = np.arange(-128, 128, dtype=np.int8).reshape(1, 256)
    for scale in (np.float32(1.0), np.float32(1.0 / 127), np.float32(0.7071), np.float32(2.0 ** -140)):
        d = q8.decode(c, np.array([scale], np.float32))
        for i, code in enumerate(range(-128, 128)):
            prod = np.float32(np.float32(code) * scale)
            u = int(np.array([prod], np.float32).view(np.uint32)[0])
            hi, low = u >> 16, u & 0xFFFF
            if low > 0x8000 or (low == 0x8000 and hi & 1):
                hi += 1
            assert int(d[0, i]) == (hi & 0xFFFF), (code, scale)
