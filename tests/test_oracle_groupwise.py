"""Pins for oracle/groupwise.py: plain group-wise 3- and 5-bit codes with an fp32 scale and min
per group of 32 ("二三五六位量化" page section 3.3's gemv_q3 form; section 2.2's packing).

Pins: the min-max rule on on-grid weights (exact recovery of s, m and q); the element-by-element
quantizer; the half-step bound; W_hat against exact rational arithmetic; the page's rewritten
sum s * sum(q x) + m * sum(x) against the plain sum of W_hat x; the listing's byte layout
(row stride cols * b / 8, 8 codes in 3 or 5 little-endian bytes) on a hand-worked row.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import bitstream, groupwise as gw
from workloads import laplace_weights

FMTS = ["q3g32", "q5g32"]


@pytest.mark.parametrize("fmt", FMTS)
def test_on_grid_weights_are_recovered(fmt):
    rng = np.random.default_rng(3)
    qmax = (1 << gw.BITS[fmt]) - 1
    n, k = 3, 128
    s = 2.0 ** rng.integers(-10, -5, size=(n, k // 32))
    m = -rng.integers(0, 64, size=(n, k // 32)) * 2.0 ** -9
    q = rng.integers(0, qmax + 1, size=(n, k))
    q[:, ::32], q[:, 1::32] = 0, qmax
    w = (np.repeat(s, 32, axis=1) * q + np.repeat(m, 32, axis=1)).astype(np.float32)
    qq, ss, mm = gw.quantize(fmt, w)
    assert np.array_equal(ss, s.astype(np.float32)) and np.array_equal(mm, m.astype(np.float32))
    assert np.array_equal(qq, q)
    assert np.array_equal(gw.dequantize(qq, ss, mm), w.astype(np.float64))


@pytest.mark.parametrize("fmt", FMTS)
def test_vectorized_matches_scalar_and_bound(fmt):
    w = laplace_weights(5, 256, 0.02, 4, outlier_frac=0.01)
    w[1, :32] = np.float32(0.003)                 # constant group: s at the floor, q = 0
    w[2, 32:64] = np.abs(w[2, 32:64])
    q, s, m = gw.quantize(fmt, w)
    for r in range(5):
        for g in range(8):
            qs, ss, ms = gw.quantize_group_scalar(fmt, w[r, 32 * g:32 * g + 32])
            assert qs == list(q[r, 32 * g:32 * g + 32]) and ss == s[r, g] and ms == m[r, g]
    assert s[1, 0] == gw.SCALE_FLOOR and np.all(q[1, :32] == 0)
    w_hat = gw.dequantize(q, s, m)
    step = np.repeat(s.astype(np.float64), 32, axis=1)
    assert np.all(np.abs(w_hat - w.astype(np.float64)) <= step / 2 * (1 + 1e-5) + 1e-12)


@pytest.mark.parametrize("fmt", FMTS)
def test_w_hat_exact_and_listing_sum(fmt):
    w = laplace_weights(2, 64, 0.02, 5)
    codes, s, m = gw.encode(fmt, w)
    q = bitstream.unpack_bits(codes, gw.BITS[fmt], 64)
    w_hat = gw.decode(fmt, codes, s, m, 64)
    for r in range(2):
        for c in range(64):
            assert Fraction(w_hat[r, c]) == Fraction(float(s[r, c // 32])) * int(q[r, c]) + Fraction(float(m[r, c // 32]))
    x = np.random.default_rng(6).standard_normal(64).astype(np.float16)
    for r in range(2):
        plain = sum(Fraction(w_hat[r, c]) * Fraction(float(x[c])) for c in range(64))
        assert gw.gemv_listing_form(bytes(codes[r]), x, fmt, s[r], m[r]) == plain


def test_listing_byte_layout_3bit():
    """Codes 0..7 of one group of 8: the 24-bit word is sum i << 3i = 0xFAC688, bytes
    88 C6 FA; the second row starts at cols * 3 / 8 bytes."""
    q = np.zeros((2, 64), np.uint8)
    q[0, :8] = np.arange(8)
    q[1, :8] = np.arange(8)[::-1]
    packed = bitstream.pack_bits(q, 3)
    assert packed.shape == (2, 24)
    assert bytes(packed[0, :3]) == bytes([0x88, 0xC6, 0xFA])
    v = int(packed[1, 0]) | (int(packed[1, 1]) << 8) | (int(packed[1, 2]) << 16)
    assert [(int(v) >> (3 * i)) & 7 for i in range(8)] == list(range(8))[::-1]


def test_zero_minimum_is_stored_as_positive_zero():
    """A group whose minimum is a zero stores +0, whichever signed zero came first."""
    w = np.zeros((2, 64), np.float32)
    w[0, :32] = np.float32(-0.0)
    w[0, 5] = np.float32(0.25)
    w[1, 40] = np.float32(-0.0)
    w[1, 41] = np.float32(0.5)
    for fmt in FMTS:
        _, s, m = gw.quantize(fmt, w)
        assert np.all(m.view(np.uint32) == 0), (fmt, m)
        for r in range(2):
            for g in range(2):
                _, ss, ms = gw.quantize_group_scalar(fmt, w[r, 32 * g:32 * g + 32])
                assert np.float32(ms).view(np.uint32) == 0


def test_bytes_and_errors():
    assert gw.algorithmic_bytes("q3g32", 2, 128) == 2 * (48 + 32)
    assert gw.algorithmic_bytes("q5g32", 2, 128) == 2 * (80 + 32)
    with pytest.raises(ValueError):
        gw.quantize("q3g32", np.zeros((1, 96), np.float32))
    bad = np.zeros((1, 64), np.float32)
    bad[0, 1] = np.nan
    with pytest.raises(ValueError):
        gw.quantize("q5g32", bad)
