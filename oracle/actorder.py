"""Act-order (column-permuted) quantized weights, by definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "二三五六位量化" page, section 2.4 (GPTQ quantizes a weight matrix column by column,
visiting the columns in order of activation importance, and that order is kept with the
weights) and section 3.2, stage 3 (the permutation index is saved with the quantized file
and restored at inference).

Reading (the pages state the idea, not the storage convention): the quantizer sees the
columns in the permuted order, so stored column c is original column perm[c]. With W_s the
dequantized stored matrix, the effective weights are W_eff[:, perm[c]] = W_s[:, c], and the
layer computes y = W_eff x. The choice of perm itself (ordering by the calibration
Hessian's diagonal) needs calibration activations and is out of scope; perm is an input.

Parity status: pinned by tests/test_oracle_actorder.py (identity permutation; weights on the
quantization grid, where quantizing the permuted matrix is exact and scattering the stored
columns back must give the original matrix for any permutation; brute force on tiny inputs).
"""
from __future__ import annotations

import numpy as np


def check_perm(perm: np.ndarray, k: int) -> np.ndarray:
    """perm as int64, after checking that it is a permutation of 0..k-1."""
    p = np.asarray(perm).astype(np.int64)
    if p.shape != (k,) or not np.array_equal(np.sort(p), np.arange(k)):
        raise ValueError("perm must be a permutation of 0..k-1")
    return p


def stored_matrix(w: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """The matrix the quantizer is given: column c of it is column perm[c] of W."""
    p = check_perm(perm, w.shape[1])
    return np.ascontiguousarray(w[:, p])


def effective_weights(w_stored_hat: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Scatter the stored (dequantized) columns back to their original positions."""
    n, k = w_stored_hat.shape
    p = check_perm(perm, k)
    w_eff = np.zeros((n, k), np.float64)
    for c in range(k):
        w_eff[:, p[c]] = w_stored_hat[:, c]
    return w_eff
