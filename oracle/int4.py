"""INT4 symmetric group formats: group 32 ("q4g32"), and groups of 16, 64 and 128 ("q4g16",
"q4g64", "q4g128").

Source: DBHOO-CIM page.
  * Section 2.1 / 3.1: symmetric quantization with scale = max|w| / 8 per group and
    q = clamp(round(w / scale), -8, 7); the page's ``quantize_group`` floors the scale at
    1e-12 and uses torch.round (round half to even) on fp32 tensors.
  * Section 3.1 (text after the code): a group is 32 consecutive elements of the
    input dimension, i.e. a contiguous slice of one row of W [out_features, in_features].
  * Section 3.2: two codes per byte, the first weight in the low nibble, stored unsigned
    0..15; decoding subtracts the sign offset to get back to [-8, 7].
  * Section 4.1: 16 bytes per group of 32 codes; scales are fp32 in a separate array
    indexed by group number.

Readings:
  * Round and clamp commute (integer bounds, monotone maps), so the two orders the page
    prints (section 2.1 vs 3.1) agree.
  * The unsigned nibble is offset binary u = q + 8 (the text says "subtract the sign
    offset"; the section 4.2 comment maps [0, 15] to [-8, 7]).
  * The page computes in fp32 (PyTorch fp32 tensors). The scale, the quotient w / scale
    and the round therefore happen in fp32 here too, so that every integer decision is
    taken in the page's precision. A group whose max|w| / 8 is below 1e-12 gets the
    scale fp32(1e-12), as the page's max(scale, 1e-12) gives.
  * K must be a multiple of the group (the page's flattened reshape would otherwise straddle
    rows).
  * Other group sizes: section 5.1 of the same page advises groups of 16 when a model has
    many outlier weights (a smaller group confines an outlier's scale to fewer weights);
    groups of 64 and 128 are the coarser end of the same trade. Everything else is the
    group-32 format with G in place of 32: codes are packed the same way and each group has
    one fp32 scale max|w| / 8, so a group costs G/2 + 4 bytes.
  * With scale = max|w| / 8, a group's largest positive weight maps to +8 and clamps to 7,
    so its error is a full scale; the page's section 3.1 remarks on this asymmetry.
    Everything else is within half a scale.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from . import bitstream

GROUP = 32
GROUPS = (16, 32, 64, 128)
SCALE_FLOOR = np.float32(1e-12)


def quantize(w: np.ndarray, group: int = GROUP) -> Tuple[np.ndarray, np.ndarray]:
    """fp32 W [n, k] -> (q int8 [n, k] in [-8, 7], scale fp32 [n, k/group])."""
    w = np.asarray(w)
    if w.dtype != np.float32 or w.ndim != 2:
        raise TypeError("W must be a 2-D float32 array")
    if group not in GROUPS:
        raise ValueError("group must be 16, 32, 64 or 128")
    n, k = w.shape
    if k % group:
        raise ValueError("K must be a multiple of the group")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    g = w.reshape(n, k // group, group)
    amax = np.abs(g).max(axis=2) if k else np.zeros((n, 0), np.float32)
    scale = (amax / np.float32(8.0)).astype(np.float32)
    scale = np.maximum(scale, SCALE_FLOOR)
    ratio = (g / scale[..., None]).astype(np.float32)          # fp32 quotient
    q = np.clip(np.rint(ratio), -8, 7).astype(np.int8)          # half to even
    return q.reshape(n, k), scale


def quantize_group_scalar(w32) -> Tuple[list, np.float32]:
    """One group, element by element (reference for the vectorized quantizer)."""
    vals = [np.float32(v) for v in w32]
    amax = np.float32(0.0)
    for v in vals:
        a = np.float32(abs(v))
        if a > amax:
            amax = a
    scale = np.float32(amax / np.float32(8.0))
    if scale < SCALE_FLOOR:
        scale = SCALE_FLOOR
    q = []
    for v in vals:
        r = np.float32(v / scale)
        qi = int(np.rint(r))
        q.append(min(7, max(-8, qi)))
    return q, scale


def pack_codes(q: np.ndarray) -> np.ndarray:
    """int8 [n, k] -> uint8 [n, k/2]: u = q + 8, byte j = u[2j] | u[2j+1] << 4."""
    u = (q.astype(np.int16) + 8).astype(np.uint8)
    return bitstream.pack_bits(u, 4)


def unpack_codes(codes: np.ndarray, k: int) -> np.ndarray:
    """uint8 [n, k/2] -> int8 [n, k]."""
    return (bitstream.unpack_bits(codes, 4, k).astype(np.int16) - 8).astype(np.int8)


def encode(w: np.ndarray, group: int = GROUP) -> Tuple[np.ndarray, np.ndarray]:
    """fp32 W -> canonical (codes uint8 [n, k/2], scales fp32 [n, k/group])."""
    q, s = quantize(w, group)
    return pack_codes(q), s


def dequantize(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """W_hat[r, c] = q[r, c] * scale[r, c // G] in fp64 (exact: 4-bit x 24-bit); the group G
    is k / scale.shape[1]."""
    n, k = q.shape
    group = k // scale.shape[1] if scale.shape[1] else GROUP
    s = np.repeat(scale.astype(np.float64), group, axis=1)
    return q.astype(np.float64) * s


def decode(codes: np.ndarray, scales: np.ndarray, k: int) -> np.ndarray:
    """Canonical encoding -> W_hat fp64 [n, k]."""
    return dequantize(unpack_codes(codes, k), scales)


def algorithmic_bytes(n: int, k: int, group: int = GROUP) -> int:
    """group/2 bytes of codes + 4 bytes of fp32 scale per group."""
    return n * (k // group) * (group // 2 + 4)
