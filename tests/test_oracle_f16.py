"""Pins the oracle's binary16 codec (the storage format of the Q8_0 scale) against numpy's
float16 conversion, an independent implementation of the same IEEE format."""
import numpy as np


def test_decode_every_bit_pattern(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = orc.f16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _finite_f16_values():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    keep = np.isfinite(vals)
    return bits[keep], vals[keep].astype(np.float32)


def test_encode_exact_values(orc):
    bits, vals = _finite_f16_values()
    assert np.array_equal(orc.f32_to_f16(vals), bits)


def test_encode_midpoints_and_neighbours(orc):
    # midpoints between consecutive positive binary16 values need 12 significant bits, so they
    # are exact float32 values; ties must go to the even neighbour, the float32 values one ulp
    # either side must go to the nearer neighbour.
    pos = np.arange(0, 0x7c00, dtype=np.uint32).astype(np.uint16).view(np.float16)
    lo = pos[:-1].astype(np.float64)
    hi = pos[1:].astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(np.inf))
    for x in (mid, below, above, -mid, -below, -above):
        assert np.array_equal(orc.f32_to_f16(x), x.astype(np.float16).view(np.uint16))


def test_encode_random_and_extremes(orc):
    rng = np.random.default_rng(7)
    e = rng.uniform(-30, 17, size=400_000)
    x = (np.sign(rng.standard_normal(e.size)) * np.exp2(e)).astype(np.float32)
    extra = np.float32([0.0, -0.0, 65504, 65519.996, 65520, 1e30, -1e30, np.inf, -np.inf,
                        2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26,
                        2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -12), 1 / 127, 4 / 127])
    x = np.concatenate([x, extra])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(orc.f32_to_f16(x), ref)
