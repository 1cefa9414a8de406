"""Pins for oracle/gemv.py (y = W_hat x, Y = X W_hat^T in fp64).

Pins: exact rational brute force on tiny non-square inputs (catches a transposed operand
or a dropped row); one-hot x selects a column exactly; zero x gives exactly zero;
linearity in x; the Sigma-x factorization of the "二三五六位量化" page, section 3.3
(sum (s*q + m) x = s * (q . x) + m * sum x) holds for decoded groups; the GEMM form equals
stacked GEMVs.
"""
import numpy as np
import pytest

from oracle import gemv, int4
from oracle import superblock as sb
from workloads import activations, laplace_weights


def _decoded(fmt, n, k, seed):
    w = laplace_weights(n, k, 0.02, seed)
    if fmt == "q4g32":
        codes, s = int4.encode(w)
        return int4.decode(codes, s, k)
    return sb.decode(fmt, sb.encode(fmt, w))


@pytest.mark.parametrize("fmt", ["q4g32", "q2sb", "q3sb", "q5sb", "q6sb"])
def test_brute_force_tiny(fmt):
    for n, k in ((3, 256), (4, 512)):
        w_hat = _decoded(fmt, n, k, seed=n * 10 + k)
        x = activations(1, k, seed=k + n)[0]
        y = gemv.gemv(w_hat, x)
        exact = gemv.gemv_exact(w_hat, x)
        assert y.shape == (n,)
        for r in range(n):
            assert abs(y[r] - float(exact[r])) <= 1e-12 * float(gemv.abs_sum(w_hat, x)[r])


def test_one_hot_zero_linearity():
    w_hat = _decoded("q3sb", 5, 512, 3)
    for col in (0, 1, 255, 256, 511):
        e = np.zeros(512, np.float16)
        e[col] = 1.0
        assert np.array_equal(gemv.gemv(w_hat, e), w_hat[:, col])
    assert np.all(gemv.gemv(w_hat, np.zeros(512, np.float16)) == 0.0)
    a = activations(1, 512, 1)[0].astype(np.float64)
    b = activations(1, 512, 2)[0].astype(np.float64)
    lhs = gemv.gemv(w_hat, 2.0 * a - b)
    rhs = 2.0 * gemv.gemv(w_hat, a) - gemv.gemv(w_hat, b)
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-12)


def test_gemm_is_stacked_gemv():
    w_hat = _decoded("q5sb", 7, 256, 8)
    xm = activations(3, 256, 9)
    y = gemv.gemm(w_hat, xm)
    assert y.shape == (3, 7)
    for m in range(3):
        assert np.allclose(y[m], gemv.gemv(w_hat, xm[m]), rtol=0, atol=1e-13)
    assert np.allclose(gemv.abs_sum(w_hat, xm)[1], gemv.abs_sum(w_hat, xm[1]), rtol=1e-15)


def test_sigma_x_factorization_q2sb():
    """section 3.3: sum_i (s*q_i - m) x_i == s * sum q_i x_i - m * sum x_i per sub-block."""
    w = laplace_weights(2, 256, 0.02, 12)
    f = sb.quantize("q2sb", w)
    x = activations(1, 256, 13)[0].astype(np.float64)
    w_hat = sb.dequantize_fields("q2sb", f)
    for r in range(2):
        total = 0.0
        for j in range(16):
            s = float(f["d"][r, 0]) * int(f["sc"][r, 0, j])
            mm = float(f["dmin"][r, 0]) * int(f["m"][r, 0, j])
            q = f["codes"][r, 0, 16 * j:16 * j + 16].astype(np.float64)
            xs = x[16 * j:16 * j + 16]
            total += s * float(q @ xs) - mm * float(xs.sum())
        assert abs(total - float(w_hat[r] @ x)) <= 1e-12 * float(np.abs(w_hat[r]) @ np.abs(x))


def test_tolerance_helper():
    y_ref = np.array([1.0, -2.0])
    bound = np.array([10.0, 10.0])
    ok = gemv.within_tolerance(np.array([1.0 + 0.019, -2.0 - 0.021]), y_ref, bound)
    assert ok.tolist() == [True, False]
