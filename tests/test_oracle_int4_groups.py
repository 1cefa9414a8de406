"""Pins for the INT4 group sizes 16, 64 and 128 in oracle/int4.py (DBHOO-CIM page, section 5.1:
smaller groups against outlier weights; the group-32 rules otherwise)."""
import numpy as np
import pytest

from oracle import int4
from workloads import laplace_weights


@pytest.mark.parametrize("group", [16, 64, 128])
def test_vectorized_matches_scalar_per_group(group):
    rng = np.random.default_rng(group)
    w = (rng.laplace(0, 0.02, size=(3, 4 * group)) * rng.choice([1, 1, 20], size=(3, 4 * group))).astype(np.float32)
    q, s = int4.quantize(w, group)
    assert s.shape == (3, 4)
    for r in range(3):
        for g in range(4):
            qs, ss = int4.quantize_group_scalar(w[r, group * g:group * (g + 1)])
            assert ss == s[r, g] and list(q[r, group * g:group * (g + 1)]) == qs


def test_bytes_per_weight():
    # group/2 code bytes + one fp32 scale per group: 6.0, 5.0, 4.5 and 4.25 bits per weight
    for group, bpw in ((16, 6.0), (32, 5.0), (64, 4.5), (128, 4.25)):
        assert int4.algorithmic_bytes(1, 4096, group) * 8 / 4096 == bpw


def test_halves_with_equal_maxima_quantize_like_group_32():
    """When both 16-weight halves of every 32-group share the same max|w|, groups of 16 have
    the group-32 scale and codes (a check of the group indexing)."""
    rng = np.random.default_rng(3)
    w = rng.uniform(-1, 1, size=(4, 128)).astype(np.float32)
    w[:, ::16] = 1.5                                   # the max of every 16-weight half
    q16, s16 = int4.quantize(w, 16)
    q32, s32 = int4.quantize(w, 32)
    assert np.array_equal(q16, q32)
    assert np.array_equal(s16, np.repeat(s32, 2, axis=1))
    # a group of 64 / 128 built from two / four such groups keeps them too
    q64, s64 = int4.quantize(w, 64)
    assert np.array_equal(q64, q32) and np.array_equal(np.repeat(s64, 2, axis=1), s32)


def test_smaller_groups_contain_outliers():
    """The page's advice: with outlier weights, groups of 16 cut the error of the weights that
    share a scale with an outlier. On Laplace weights with 0.1% x20 outliers the mean
    absolute error falls as the group shrinks."""
    w = laplace_weights(64, 1024, 0.02, 11, outlier_frac=0.001)
    err = {}
    for group in (16, 32, 64, 128):
        q, s = int4.quantize(w, group)
        err[group] = float(np.mean(np.abs(int4.dequantize(q, s) - w.astype(np.float64))))
    assert err[16] < err[32] < err[64] < err[128]


def test_error_bound_any_group():
    w = laplace_weights(8, 512, 0.02, 5, outlier_frac=0.01)
    for group in (16, 64, 128):
        q, s = int4.quantize(w, group)
        sc = np.repeat(s.astype(np.float64), group, axis=1)
        err = np.abs(int4.dequantize(q, s) - w.astype(np.float64))
        tail = w.astype(np.float64) > 7.5 * sc       # the clamped positive tail: error up to one scale
        assert np.all(err[~tail] <= sc[~tail] / 2 * (1 + 1e-6))
        assert np.all(err[tail] <= sc[tail] * (1 + 1e-6))


def test_rejects_bad_group_and_k():
    with pytest.raises(ValueError):
        int4.quantize(np.zeros((1, 64), np.float32), 48)
    with pytest.raises(ValueError):
        int4.quantize(np.zeros((1, 64), np.float32), 128)
