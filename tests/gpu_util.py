"""Helpers for the GPU parity tests: the oracle side and the device side, kept apart."""
import numpy as np

import dequant_gemv_q4g32_amd as qg
from oracle import gemv as ogemv
from oracle import groupwise as gw
from oracle import int4
from oracle import superblock as sb


def oracle_decode(fmt, w):
    """Oracle's own quantization of fp32 W: (logical codes uint8 [n, k], W_hat fp64 [n, k])."""
    n, k = w.shape
    if fmt in qg.Q4_GROUPS:
        q, s = int4.quantize(w, qg.Q4_GROUPS[fmt])
        return (q.astype(np.int16) + 8).astype(np.uint8), int4.dequantize(q, s)
    if fmt == "q4g32h":
        q, s16 = int4.quantize_h(w)
        return (q.astype(np.int16) + 8).astype(np.uint8), int4.dequantize(q, s16.astype(np.float32))
    if fmt in gw.BITS:
        q, s, m = gw.quantize(fmt, w)
        return q, gw.dequantize(q, s, m)
    if fmt == "q4a32":
        q, s, z = int4.quantize_asym(w)
        return q, int4.dequantize_asym(q, s, z)
    f = sb.quantize(fmt, w)
    return f["codes"].reshape(n, k), sb.dequantize_fields(fmt, f)


def oracle_y(w_hat, xm):
    """Reference outputs and the per-output tolerance scale sum |w_hat * x|."""
    return ogemv.gemm(w_hat, xm), ogemv.abs_sum(w_hat, xm)


def assert_close(y, y_ref, bound, what=""):
    y = np.asarray(y, np.float64)
    ok = ogemv.within_tolerance(y, y_ref, bound)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} outputs out of tolerance, e.g. "
                             + ", ".join(f"{tuple(i)}: got {y[tuple(i)]:.6g} want {y_ref[tuple(i)]:.6g} "
                                         f"bound {ogemv.REL_TOL * bound[tuple(i)]:.3g}" for i in idx))


def device_weights(fmt, w):
    n, k = w.shape
    return qg.to_device(fmt, qg.quantize(fmt, w), n, k)
