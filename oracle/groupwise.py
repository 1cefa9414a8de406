"""Plain group-wise 3-bit and 5-bit formats with a scale and a min per group of 32 ("q3g32",
"q5g32"): the form of the scalar dequant GEMV that the "二三五六位量化" page prints.

Source: "二三五六位量化" page.
  * Section 3.3: the scalar skeleton ``gemv_q3(w, x, y, rows, cols, group, scales, mins)``:
    row r's codes start at r * (cols * 3 / 8) bytes, every 8 codes sit in 3 bytes read as a
    24-bit little-endian word (code i at bits 3i..3i+2), group g = c / group has the fp32
    scale s and min m, and the weight is s * q + m; the text that follows rewrites the sum as
    s * sum(q x) + m * sum(x).
  * Section 2.2: the same little-endian packing for 5-bit codes, 8 codes in 5 bytes.
  * Section 2.1: the 3-bit tier works with groups of 32; the 5- and 6-bit tiers need no more
    than groups of 32 and may use a plain single-level scale.

Readings (the page gives the decoding, not the quantizer):
  * Groups of 32 consecutive weights of a row (section 2.1), each with its own scale and min;
    the listing indexes ``scales[g]`` with g = c / group only, which read literally would
    share the scales across rows: taken as a per-row array [rows][cols / group], the layout
    every other quantizer on the pages uses.
  * Min-max rule in fp32 (the listing's float scales): m = min w, s = (max w - min w) / (2^b - 1)
    floored at 1e-12 (the INT4 page's floor), q = clamp(rint((w - m) / s), 0, 2^b - 1) with the
    difference and the quotient each rounded to fp32. A group whose minimum is a zero stores
    +0 (m + 0 in fp32): the minimum of +0 and -0 is otherwise either, by reduction order. w_hat = s * q + m (computed exactly in
    fp64 here). Every weight is then within s / 2 of w_hat, up to the fp32 rounding of the
    difference and the quotient.
  * Canonical encoding: the codes of a row as one little-endian bitstream of b-bit codes
    (cols * b / 8 bytes, the listing's row stride), then fp32 scales [n][k/32], then fp32
    mins [n][k/32]. K is a multiple of 64 (whole device units).
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

from . import bitstream

GROUP = 32
BITS = {"q3g32": 3, "q5g32": 5}
SCALE_FLOOR = np.float32(1e-12)


def quantize(fmt: str, w: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """fp32 W [n, k] -> (q uint8 [n, k], scale fp32 [n, k/32], min fp32 [n, k/32])."""
    b = BITS[fmt]
    w = np.asarray(w)
    if w.dtype != np.float32 or w.ndim != 2:
        raise TypeError("W must be a 2-D float32 array")
    n, k = w.shape
    if k % 64:
        raise ValueError("K must be a multiple of 64")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    g = w.reshape(n, k // GROUP, GROUP)
    lo = g.min(axis=2) if k else np.zeros((n, 0), np.float32)
    hi = g.max(axis=2) if k else np.zeros((n, 0), np.float32)
    qmax = (1 << b) - 1
    s = ((hi - lo) / np.float32(qmax)).astype(np.float32)
    if not np.all(np.isfinite(s)):
        raise OverflowError("a group's range does not fit fp32")
    s = np.maximum(s, SCALE_FLOOR)
    lo = (lo + np.float32(0.0)).astype(np.float32)       # -0 -> +0
    diff = (g - lo[..., None]).astype(np.float32)
    r = (diff / s[..., None]).astype(np.float32)
    q = np.clip(np.rint(r), 0, qmax).astype(np.uint8)
    return q.reshape(n, k), s, lo


def quantize_group_scalar(fmt: str, w32) -> Tuple[List[int], np.float32, np.float32]:
    """One group, element by element (reference for the vectorized quantizer)."""
    qmax = (1 << BITS[fmt]) - 1
    vals = [np.float32(v) for v in w32]
    lo, hi = vals[0], vals[0]
    for v in vals[1:]:
        lo = min(lo, v)
        hi = max(hi, v)
    s = np.float32(np.float32(hi - lo) / np.float32(qmax))
    if s < SCALE_FLOOR:
        s = SCALE_FLOOR
    lo = np.float32(lo + np.float32(0.0))
    q = []
    for v in vals:
        r = np.float32(np.float32(v - lo) / s)
        q.append(int(min(qmax, max(0, int(np.rint(r))))))
    return q, s, np.float32(lo)


def dequantize(q: np.ndarray, s: np.ndarray, m: np.ndarray) -> np.ndarray:
    """W_hat = s * q + m in fp64. Exact when the product and the min lie within fp64's
    53 bits of each other (asserted)."""
    ss = np.repeat(s.astype(np.float64), GROUP, axis=1)
    mm = np.repeat(m.astype(np.float64), GROUP, axis=1)
    prod = ss * q.astype(np.float64)                  # exact: 24-bit x 5-bit
    out = prod + mm
    assert np.array_equal(out - mm, prod), "w_hat not exact in fp64"
    return out


def encode(fmt: str, w: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """fp32 W -> canonical (codes uint8 [n, k*b/8], scales fp32 [n, k/32], mins fp32 [n, k/32])."""
    q, s, m = quantize(fmt, w)
    return bitstream.pack_bits(q, BITS[fmt]), s, m


def decode(fmt: str, codes: np.ndarray, s: np.ndarray, m: np.ndarray, k: int) -> np.ndarray:
    """Canonical encoding -> W_hat fp64 [n, k]."""
    return dequantize(bitstream.unpack_bits(codes, BITS[fmt], k), s, m)


def gemv_listing_form(codes_row: bytes, x, fmt: str, s_row, m_row) -> float:
    """One output of the page's scalar form for one row, in exact rational arithmetic: for each
    group, s * sum(q x) + m * sum(x) over codes read from the little-endian stream (small
    inputs only)."""
    from fractions import Fraction
    b = BITS[fmt]
    k = len(x)
    q = bitstream.unpack_bits_scalar(codes_row, b, k)
    acc = Fraction(0)
    for g in range(k // GROUP):
        qx = sum(Fraction(int(q[c])) * Fraction(float(x[c])) for c in range(GROUP * g, GROUP * g + GROUP))
        sx = sum(Fraction(float(x[c])) for c in range(GROUP * g, GROUP * g + GROUP))
        acc += Fraction(float(s_row[g])) * qx + Fraction(float(m_row[g])) * sx
    return acc


def algorithmic_bytes(fmt: str, n: int, k: int) -> int:
    """Codes (b/8 bytes per weight) plus a 4-byte scale and a 4-byte min per group of 32."""
    return n * (k * BITS[fmt] // 8 + (k // GROUP) * 8)
