"""Pins the oracle's Q8_0 codec ("Core Architecture & The 4-Brick Pipeline", Sec. 5, block_q8_0:
32 int8 values plus an FP16 scale in 34 bytes, 8-bit symmetric) to facts fixed by the format and
by arithmetic, not to a second copy of its own formula."""
from decimal import ROUND_HALF_UP, Decimal

import numpy as np
import pytest


def f16_bits(x: float) -> int:
    return int(np.float16(x).view(np.uint16))


def half_away(x: float) -> int:
    """Nearest integer, halves away from zero (Decimal's ROUND_HALF_UP on the exact value)."""
    return int(Decimal(float(x)).quantize(Decimal(1), rounding=ROUND_HALF_UP))


def split(b):
    """bytes of one block -> (scale bits, int8 values)."""
    b = np.asarray(b, dtype=np.uint8)
    return int(b[0]) | int(b[1]) << 8, b[2:34].view(np.int8).astype(np.int64)


def test_block_size_is_34_bytes(orc):
    x = np.ones((5, 64), dtype=np.float32)
    out = orc.q8_0_pack(x)
    assert out.shape == (5, 68)  # 2 blocks x 34 bytes per 64-dim row
    # 34 bytes per 32 values against 64 for FP16: the pages' 46.88 % reduction
    assert round((1 - 34 / 64) * 100, 2) == 46.88


def test_exact_scale_blocks_round_half_away(orc):
    """amax = 127 * s for a binary16 value s gives d = s exactly, so the stored scale is s and
    every q is x / s rounded to nearest with halves away from zero.  Values (k + 1/2) * s are
    exact ties."""
    rng = np.random.default_rng(11)
    scales = [1.0, 0.5, 2.0 ** -7, 0.0078735352, 0.02392578, 1.5, 3.0, 0.0311279296875]
    for s in scales:
        s = float(np.float16(s))  # make it a binary16 value
        k = rng.integers(-126, 126, size=32)
        half = rng.random(32) < 0.5
        vals = (k + np.where(half, 0.5, 0.0)) * s
        vals[rng.integers(0, 32)] = -127 * s if rng.random() < 0.5 else 127 * s
        x = vals.astype(np.float32)
        assert np.array_equal(x.astype(np.float64), vals)  # exact in float32
        d_bits, q = split(orc.q8_0_pack(x))
        assert d_bits == f16_bits(s)
        want = [half_away(v / s) for v in vals]
        assert q.tolist() == want, s


def test_scale_stored_little_endian_first(orc):
    x = np.zeros(64, dtype=np.float32)
    x[3] = 127.0   # block 0: scale 1.0 = 0x3c00
    x[40] = -254.0  # block 1: scale 2.0 = 0x4000
    b = orc.q8_0_pack(x)
    assert b[:2].tolist() == [0x00, 0x3C]
    assert b[34:36].tolist() == [0x00, 0x40]
    assert b[2 + 3] == 127
    assert b[36 + 8].view(np.int8) == -127
    assert np.count_nonzero(b) == 4  # 0x3c, 0x40 and the two values


def test_zero_block(orc):
    assert not orc.q8_0_pack(np.zeros(32, dtype=np.float32)).any()


def _random_blocks(n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 32)).astype(np.float32)
    # widen the dynamic range, staying inside binary16's normal scale range
    x *= np.exp2(rng.uniform(-5, 10, size=(n, 1))).astype(np.float32)
    return x


def test_round_trip_bound(orc):
    """|x - q * d16| <= d16 * (1/2 + 2^-16): the reconstruction error stays within half a step
    of the STORED scale; the slack covers the float32 rounding of x / d16."""
    x = _random_blocks(200_000, 1)
    b = orc.q8_0_pack(x)
    y = orc.q8_0_dequant(b)
    d = orc.f16_to_f64(b[:, :2].copy().view(np.uint16)[:, 0])
    err = np.abs(x.astype(np.float64) - y)
    assert np.all(err <= d[:, None] * (0.5 + 2.0 ** -16))


def test_largest_magnitude_maps_to_127(orc):
    x = _random_blocks(50_000, 2)
    b = orc.q8_0_pack(x)
    q = b[:, 2:].view(np.int8)
    i = np.argmax(np.abs(x), axis=1)
    r = np.arange(x.shape[0])
    assert np.array_equal(q[r, i].astype(np.int64), np.where(x[r, i] > 0, 127, -127))
    assert np.abs(q.astype(np.int64)).max() <= 127  # symmetric: -128 never appears


def test_idempotent(orc):
    """Re-packing the dequantised values reproduces the bytes: the max element becomes
    127 * d16, whose division by 127 is exact, so the scale and every q come back."""
    x = _random_blocks(100_000, 3)
    b = orc.q8_0_pack(x)
    y = orc.q8_0_dequant(b).astype(np.float32)
    assert np.array_equal(orc.q8_0_dequant(b), y.astype(np.float64))  # q * d16 fits float32
    assert np.array_equal(orc.q8_0_pack(y), b)


def test_sign_symmetry(orc):
    x = _random_blocks(50_000, 4)
    b = orc.q8_0_pack(x)
    bn = orc.q8_0_pack(-x)
    assert np.array_equal(b[:, :2], bn[:, :2])
    assert np.array_equal(b[:, 2:].view(np.int8).astype(np.int64),
                          -bn[:, 2:].view(np.int8).astype(np.int64))


def test_dequant_hand_block(orc):
    blk = np.zeros(34, dtype=np.uint8)
    blk[0:2] = [0x00, 0x38]  # 0x3800 = 0.5
    q = np.array([1, -1, 127, -127, 0, 2] + [0] * 26, dtype=np.int8)
    blk[2:] = q.view(np.uint8)
    y = orc.q8_0_dequant(blk)
    assert y[:6].tolist() == [0.5, -0.5, 63.5, -63.5, 0.0, 1.0]


def test_out_of_range_rejected(orc):
    x = np.zeros(32, dtype=np.float32)
    x[0] = 1e7  # amax / 127 exceeds the largest binary16 value
    with pytest.raises(ValueError):
        orc.q8_0_pack(x)
    x[0] = np.nan
    with pytest.raises(ValueError):
        orc.q8_0_pack(x)
