"""Pins for the asymmetric INT4 groups (q4a32) in oracle/int4.py ("二三五六位量化" page section
2.1: q = round(x / s) + z, x = s (q - z); DBHOO-CIM page section 5.1)."""
import numpy as np
import pytest

from oracle import bitstream, int4
from workloads import laplace_weights


def test_vectorized_matches_scalar():
    rng = np.random.default_rng(1)
    w = (rng.laplace(0.01, 0.02, size=(4, 256)) * rng.choice([1, 1, 9], size=(4, 256))).astype(np.float32)
    w[1, :32] = np.abs(w[1, :32])            # positive-only group
    w[2, 32:64] = -np.abs(w[2, 32:64])       # negative-only group
    w[3, 64:96] = 0                          # zero group
    q, s, z = int4.quantize_asym(w)
    for r in range(4):
        for g in range(8):
            qs, ss, zs = int4.quantize_asym_group_scalar(w[r, 32 * g:32 * g + 32])
            assert ss == s[r, g] and zs == z[r, g] and list(q[r, 32 * g:32 * g + 32]) == qs


def test_on_grid_weights_are_exact():
    """w = s (q - z) with the group's range hitting both ends of [0, 15] (so the rule recovers s
    and z exactly) quantizes without error."""
    rng = np.random.default_rng(2)
    n, k = 3, 128
    s = 2.0 ** rng.integers(-8, -3, size=(n, k // 32))
    z = rng.integers(1, 15, size=(n, k // 32))
    q = rng.integers(0, 16, size=(n, k))
    q[:, ::32], q[:, 1::32] = 0, 15           # the ends of the code range in every group
    w = ((q - np.repeat(z, 32, axis=1)) * np.repeat(s, 32, axis=1)).astype(np.float32)
    qq, ss, zz = int4.quantize_asym(w)
    assert np.array_equal(ss, s.astype(np.float32)) and np.array_equal(zz, z)
    assert np.array_equal(int4.dequantize_asym(qq, ss, zz), w.astype(np.float64))


def test_zero_decodes_to_zero_and_bounds():
    w = laplace_weights(16, 512, 0.02, 3, outlier_frac=0.01) + np.float32(0.01)
    w[0, 7] = 0
    q, s, z = int4.quantize_asym(w)
    w_hat = int4.dequantize_asym(q, s, z)
    assert w_hat[0, 7] == 0.0
    assert np.all(q <= 15) and np.all(z <= 15)
    err = np.abs(w_hat - w.astype(np.float64))
    assert np.all(err <= np.repeat(s.astype(np.float64), 32, axis=1) * (1 + 1e-6))
    # most weights sit inside the grid: within half a step
    inner = err <= np.repeat(s.astype(np.float64), 32, axis=1) / 2 * (1 + 1e-6)
    assert inner.mean() > 0.99


def test_asymmetric_beats_symmetric_on_a_shifted_layer():
    """For a layer whose weights are not centred on zero, the asymmetric grid spends its 16
    levels on the range the weights occupy and the error drops (the zero point's purpose)."""
    w = (laplace_weights(32, 1024, 0.02, 4) * np.float32(0.5) + np.float32(0.03)).astype(np.float32)
    qa, sa, za = int4.quantize_asym(w)
    qs, ss = int4.quantize(w)
    ea = np.mean(np.abs(int4.dequantize_asym(qa, sa, za) - w))
    es = np.mean(np.abs(int4.dequantize(qs, ss) - w))
    assert ea < 0.8 * es


def test_encoding_and_bytes():
    w = laplace_weights(2, 128, 0.02, 5)
    codes, s, z = int4.encode_asym(w)
    q, _, _ = int4.quantize_asym(w)
    assert np.array_equal(bitstream.unpack_bits(codes, 4, 128), q)
    assert int4.algorithmic_bytes_asym(2, 128) == codes.nbytes + s.nbytes + z.nbytes == 2 * 4 * 21
    with pytest.raises(ValueError):
        int4.quantize_asym(np.zeros((1, 96), np.float32))
