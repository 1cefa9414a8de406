"""Pins for oracle/int4.py (INT4 symmetric group-32).

Pins: a hand-worked group (tests/golden/int4_group.json) covering the clamp at +8,
half-to-even in both directions, the offset-binary nibbles and the low-nibble-first byte
order; the DBHOO-CIM page's error behaviour (within scale/2, except the clamped tail
(7.5*scale, 8*scale] which is within one scale); the element-by-element quantizer against
the vectorized one; the byte count (16 B of codes + 4 B fp32 scale per 32 weights);
special cases (zero group, a lone -max weight is exact).
"""
import json
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import int4
from workloads import laplace_weights

G = json.load(open(os.path.join(GOLDEN, "int4_group.json")))


def test_hand_worked_group():
    w = np.array([G["w"]], np.float32)
    q, s = int4.quantize(w)
    assert s.shape == (1, 1) and s[0, 0] == np.float32(G["scale"])
    assert q[0].tolist() == G["q"]
    codes = int4.pack_codes(q)
    assert bytes(codes[0]) == bytes.fromhex(G["bytes"].replace(" ", ""))
    w_hat = int4.decode(codes, s, 32)
    assert w_hat[0, :8].tolist() == G["w_hat"]
    qs, ss = int4.quantize_group_scalar(G["w"])
    assert qs == G["q"] and ss == np.float32(G["scale"])


def test_zero_group():
    w = np.zeros((1, 32), np.float32)
    q, s = int4.quantize(w)
    assert s[0, 0] == np.float32(G["zero_group"]["scale_fp32_of"])
    assert bytes(int4.pack_codes(q)[0]) == bytes.fromhex(G["zero_group"]["bytes"].replace(" ", ""))
    assert np.all(int4.dequantize(q, s) == 0.0)


def test_negative_max_is_exact():
    w = np.zeros((1, 32), np.float32)
    w[0, 5] = -0.75
    q, s = int4.quantize(w)
    assert q[0, 5] == -8 and int4.dequantize(q, s)[0, 5] == -0.75


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_error_bounds_and_ranges(seed):
    w = laplace_weights(64, 512, 0.02, seed, outlier_frac=0.01)
    q, s = int4.quantize(w)
    assert q.min() >= -8 and q.max() <= 7
    w_hat = int4.dequantize(q, s)
    scale = np.repeat(s.astype(np.float64), 32, axis=1)
    err = np.abs(w_hat - w.astype(np.float64))
    tail = w.astype(np.float64) > 7.5 * scale
    slack = 1e-6 * scale                     # fp32 quotient rounding at exact halves
    assert np.all(err[~tail] <= scale[~tail] / 2 + slack[~tail])
    assert np.all(err[tail] <= scale[tail] + slack[tail])
    assert tail.sum() > 0                    # the clamped tail exists for max-positive groups


def test_vectorized_matches_scalar():
    w = laplace_weights(8, 256, 0.02, 9, outlier_frac=0.02)
    q, s = int4.quantize(w)
    for r in range(8):
        for g in range(8):
            qs, ss = int4.quantize_group_scalar(w[r, 32 * g:32 * g + 32])
            assert qs == q[r, 32 * g:32 * g + 32].tolist() and ss == s[r, g]


def test_encode_decode_round_trip_and_sizes():
    w = laplace_weights(16, 1024, 0.02, 4)
    codes, s = int4.encode(w)
    assert codes.shape == (16, 512) and codes.dtype == np.uint8
    assert s.shape == (16, 32) and s.dtype == np.float32
    q, _ = int4.quantize(w)
    assert np.array_equal(int4.unpack_codes(codes, 1024), q)
    assert int4.algorithmic_bytes(16, 1024) == codes.nbytes + s.nbytes == 16 * 32 * 20


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        int4.quantize(np.zeros((2, 48), np.float32))
    bad = np.zeros((1, 32), np.float32)
    bad[0, 3] = np.nan
    with pytest.raises(ValueError):
        int4.quantize(bad)
