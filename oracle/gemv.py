"""Dequantize-and-multiply, by definition: y = W_hat x and Y = X W_hat^T in fp64.

Source: "二三五六位量化" page, section 1.2 (decode is a [1, hidden] x [hidden, hidden]
GEMV; prefill is the same contraction with batch x seq_len rows) and section 3.3 (the scalar
``gemv_q3``: y[r] = sum_c (s*q + m) * x[c]); DBHOO-CIM page, section 2.2 (activations stay
fp16/fp32 while weights are low-bit) and section 3.3 (dequantized weights meet the
activations directly in a floating-point multiply-add).

Reading: W is [out_features, in_features] (DBHOO-CIM section 3.1 comment), so
y[r] = sum_k W_hat[r, k] * x[k] and Y[m, r] = sum_k X[m, k] * W_hat[r, k]. The dequantized
weights are exact in fp64 and x is fp16, so the only rounding here is the fp64 sum.

Tolerance (the acceptance bar for any faster implementation of the same contraction):
|y[r] - y_ref[r]| <= 2e-3 * sum_k |W_hat[r, k] * x[k]| per output.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

REL_TOL = 2e-3


def gemv(w_hat: np.ndarray, x: np.ndarray) -> np.ndarray:
    """fp64 W_hat [n, k], x [k] (fp16) -> y fp64 [n]."""
    return np.asarray(w_hat, np.float64) @ np.asarray(x, np.float64)


def gemm(w_hat: np.ndarray, xm: np.ndarray) -> np.ndarray:
    """fp64 W_hat [n, k], X [m, k] (fp16) -> Y fp64 [m, n]."""
    return np.asarray(xm, np.float64) @ np.asarray(w_hat, np.float64).T


def abs_sum(w_hat: np.ndarray, xm: np.ndarray) -> np.ndarray:
    """sum_k |W_hat[r, k] * X[m, k]|, shape [m, n] (or [n] for a vector x)."""
    xa = np.abs(np.asarray(xm, np.float64))
    wa = np.abs(np.asarray(w_hat, np.float64))
    return xa @ wa.T if xa.ndim == 2 else wa @ xa


def gemv_exact(w_hat_rows, x) -> list:
    """Exact rational y = W_hat x for tiny inputs (Fractions, element by element)."""
    out = []
    for row in w_hat_rows:
        acc = Fraction(0)
        for wv, xv in zip(row, x):
            acc += Fraction(float(wv)) * Fraction(float(xv))
        out.append(acc)
    return out


def within_tolerance(y, y_ref, bound, rel=REL_TOL):
    """Boolean mask of outputs meeting |y - y_ref| <= rel * bound."""
    return np.abs(np.asarray(y, np.float64) - np.asarray(y_ref, np.float64)) <= rel * np.asarray(bound, np.float64)
