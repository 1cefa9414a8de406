"""Pins for oracle/actorder.py (act-order weights: "二三五六位量化" page, sections 2.4 and
3.2 stage 3)."""
import numpy as np
import pytest

from oracle import actorder, int4
from oracle import gemv as ogemv


def test_identity_permutation_changes_nothing():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((5, 64))
    assert np.array_equal(actorder.stored_matrix(w, np.arange(64)), w)
    assert np.array_equal(actorder.effective_weights(w, np.arange(64)), w)


def test_on_grid_weights_round_trip_through_any_permutation():
    """The stored matrix is built on the INT4 grid: every group of 32 stored columns is s * q
    with q in [-8, 7] and one q = -8, so its scale max|w|/8 is exactly s and quantization is
    exact. The original matrix is W = effective_weights(stored, perm). Then the quantizer's
    input stored_matrix(W, perm) must be the stored matrix, its dequantization must scatter
    back to W, and W_eff x must equal W x: a swapped direction (perm^-1 for perm) or a wrong
    axis fails one of these."""
    rng = np.random.default_rng(2)
    n, k = 6, 128
    q = rng.integers(-8, 8, size=(n, k))
    q[:, ::32] = -8
    s = np.repeat(2.0 ** rng.integers(-6, 0, size=(n, k // 32)), 32, axis=1)
    stored = (q * s).astype(np.float32)
    perm = rng.permutation(k)
    w = actorder.effective_weights(stored.astype(np.float64), perm)
    assert np.array_equal(actorder.stored_matrix(w, perm), stored.astype(np.float64))
    qq, sc = int4.quantize(stored)
    w_hat = int4.dequantize(qq, sc)
    assert np.array_equal(w_hat, stored.astype(np.float64))       # exact on the grid
    w_eff = actorder.effective_weights(w_hat, perm)
    assert np.array_equal(w_eff, w)
    x = rng.standard_normal(k).astype(np.float16)
    assert np.allclose(ogemv.gemv(w_eff, x), w @ x.astype(np.float64), rtol=0, atol=1e-12)
    # the inverse permutation gives a different matrix (so the test can tell them apart)
    inv = np.argsort(perm)
    assert not np.array_equal(actorder.effective_weights(w_hat, inv), w)


def test_effective_matvec_is_the_gathered_matvec_brute_force():
    """y = W_eff x computed element by element equals W_s x[perm] on tiny inputs."""
    rng = np.random.default_rng(3)
    n, k = 3, 8
    ws = rng.standard_normal((n, k))
    x = rng.standard_normal(k)
    perm = rng.permutation(k)
    w_eff = actorder.effective_weights(ws, perm)
    for r in range(n):
        direct = sum(w_eff[r, j] * x[j] for j in range(k))
        gathered = sum(ws[r, c] * x[perm[c]] for c in range(k))
        assert abs(direct - gathered) < 1e-12
    assert np.allclose(ogemv.gemv(w_eff, x), ws @ x[perm], rtol=0, atol=1e-12)


def test_rejects_non_permutations():
    w = np.zeros((2, 4))
    for bad in ([0, 1, 2, 2], [0, 1, 2], [0, 1, 2, 4]):
        with pytest.raises(ValueError):
            actorder.stored_matrix(w, np.array(bad))
