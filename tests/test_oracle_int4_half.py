"""Pins for INT4 groups of 32 with fp16 scales (q4g32h) in oracle/int4.py ("二三五六位量化"
page section 2.1: a 16-bit scale per group of 32; DBHOO-CIM page sections 2.1 and 3.1: the
INT4 rule)."""
import numpy as np
import pytest

from oracle import bitstream, int4
from workloads import laplace_weights


def _all_finite_halves():
    bits = np.arange(0x7C00, dtype=np.uint16)                 # +0 .. largest finite
    return bits, bits.view(np.float16).astype(np.float64)


def _nearest_half_bits(v: float) -> int:
    """fp16 nearest to v >= 0 by search over every finite fp16 value; ties to the even
    significand (an independent statement of round-to-nearest-even)."""
    bits, vals = _all_finite_halves()
    d = np.abs(vals - v)
    best = np.nonzero(d == d.min())[0]
    if best.size == 1:
        return int(bits[best[0]])
    return int(bits[best[np.argmin(bits[best] & 1)]])        # even last bit


def test_scale_is_nearest_fp16_of_max_over_8():
    rng = np.random.default_rng(7)
    w = (rng.laplace(0, 1, size=(8, 64 * 8)) * 10.0 ** rng.integers(-7, 3, size=(8, 1))).astype(np.float32)
    _, s16 = int4.quantize_h(w)
    amax = np.abs(w.reshape(8, -1, 32)).max(axis=2)
    for r in range(8):
        for g in range(0, s16.shape[1], 3):
            s32 = float(np.float32(amax[r, g] / np.float32(8)))
            want = _nearest_half_bits(s32)
            want = want if want else 1                        # the 2^-24 floor
            assert int(s16[r, g:g + 1].view(np.uint16)[0]) == want, (r, g, s32)


def test_codes_against_the_stored_scale():
    """q = clamp(rint(w / s), -8, 7) with s the stored fp16 value, checked element by element
    with Python floats (w / s in fp32 is the correctly rounded quotient)."""
    w = laplace_weights(3, 128, 0.02, 8, outlier_frac=0.02)
    q, s16 = int4.quantize_h(w)
    for r in range(3):
        for c in range(128):
            s = float(s16[r, c // 32])
            ratio = float(np.float32(np.float32(w[r, c]) / np.float32(s)))
            assert q[r, c] == min(7, max(-8, int(np.rint(ratio))))


def test_on_grid_weights_are_exact():
    rng = np.random.default_rng(9)
    n, k = 4, 256
    s = (2.0 ** rng.integers(-12, -4, size=(n, k // 32))).astype(np.float64)
    q = rng.integers(-8, 8, size=(n, k))
    q[:, ::32] = -8                                           # max|w| = 8 s in every group
    w = (q * np.repeat(s, 32, axis=1)).astype(np.float32)
    qq, ss = int4.quantize_h(w)
    assert np.array_equal(ss.astype(np.float64), s) and np.array_equal(qq, q)
    assert np.array_equal(int4.dequantize(qq, ss.astype(np.float32)), w.astype(np.float64))


def test_error_bound_floor_and_overflow():
    w = laplace_weights(16, 1024, 0.02, 10, outlier_frac=0.01)
    w[0, :32] = np.float32(1e-9)                              # scale rounds to 0: floor 2^-24
    q, s16 = int4.quantize_h(w)
    assert s16[0, 0] == np.float16(2.0 ** -24) and np.all(q[0, :32] == 0)
    s = np.repeat(s16.astype(np.float64), 32, axis=1)
    err = np.abs(int4.dequantize(q, s16.astype(np.float32)) - w.astype(np.float64))
    assert np.all(err <= s * 1.01 + 1e-9)                     # clamped +8 -> 7: about one scale
    inside = w.astype(np.float64) / s < 7.5                  # not clamped at the top
    assert np.all(err[inside] <= s[inside] / 2 * (1 + 1e-6))
    assert inside.mean() > 0.97
    big = np.zeros((1, 64), np.float32)
    big[0, 3] = np.float32(6e5)                               # 6e5 / 8 > 65504
    with pytest.raises(OverflowError):
        int4.quantize_h(big)


def test_encoding_and_bytes():
    w = laplace_weights(2, 128, 0.02, 11)
    codes, s16 = int4.encode_h(w)
    q, _ = int4.quantize_h(w)
    assert np.array_equal(int4.unpack_codes(codes, 128), q)
    assert int4.algorithmic_bytes_h(2, 128) == codes.nbytes + s16.nbytes == 2 * 4 * 18
    with pytest.raises(ValueError):
        int4.quantize_h(np.zeros((1, 96), np.float32))
