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


# ---- asymmetric INT4, groups of 32 ("q4a32") -----------------------------------------------
#
# Source: "二三五六位量化" page, section 2.1 (linear quantization q = round(x / s) + z,
# x = s (q - z): symmetric sets z = 0, asymmetric keeps the zero point z, which matters more the
# fewer levels there are) and DBHOO-CIM page, section 5.1 (a layer whose largest weights stand
# out from the rest may need asymmetric quantization instead of the symmetric grid).
#
# Readings (the pages give the formula, not the range rule or the storage):
#   * the group range includes zero: lo = min(0, min w), hi = max(0, max w), so that a zero
#     weight decodes to exactly zero; s = max((hi - lo) / 15, 1e-12); z = clamp(rint(-lo / s),
#     0, 15); q = clamp(rint(w / s) + z, 0, 15); w_hat = s * (q - z). All in fp32 with rint
#     half-to-even, as the symmetric INT4 quantizer computes;
#   * storage: the unsigned codes q (two per byte, first weight in the low nibble), fp32
#     scales [n][k/32] and uint8 zero points [n][k/32]: 21 bytes per group (5.25 bpw);
#   * K a multiple of 64 (whole lane units).
# Error: within s/2 inside the grid; the rounding of z moves the grid by at most s/2, so a
# group's extreme weight can be clipped by up to s/2 more (within s).

ASYM_QMAX = 15


def quantize_asym(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """fp32 W [n, k] (k % 64 == 0) -> (q uint8 [n, k] in [0, 15], scale fp32 [n, k/32],
    zero point uint8 [n, k/32])."""
    w = np.asarray(w)
    if w.dtype != np.float32 or w.ndim != 2:
        raise TypeError("W must be a 2-D float32 array")
    n, k = w.shape
    if k % 64:
        raise ValueError("K must be a multiple of 64")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    g = w.reshape(n, k // GROUP, GROUP)
    lo = np.minimum(np.float32(0), g.min(axis=2) if k else np.zeros((n, 0), np.float32)).astype(np.float32)
    hi = np.maximum(np.float32(0), g.max(axis=2) if k else np.zeros((n, 0), np.float32)).astype(np.float32)
    s = ((hi - lo) / np.float32(ASYM_QMAX)).astype(np.float32)
    s = np.maximum(s, SCALE_FLOOR)
    z = np.clip(np.rint((-lo / s).astype(np.float32)), 0, ASYM_QMAX).astype(np.uint8)
    r = (g / s[..., None]).astype(np.float32)
    q = np.clip(np.rint(r) + z[..., None].astype(np.float32), 0, ASYM_QMAX).astype(np.uint8)
    return q.reshape(n, k), s, z


def quantize_asym_group_scalar(w32):
    """One group, element by element (reference for the vectorized quantizer)."""
    vals = [np.float32(v) for v in w32]
    lo, hi = np.float32(0.0), np.float32(0.0)
    for v in vals:
        lo = min(lo, v)
        hi = max(hi, v)
    s = np.float32(np.float32(hi - lo) / np.float32(ASYM_QMAX))
    if s < SCALE_FLOOR:
        s = SCALE_FLOOR
    z = int(min(ASYM_QMAX, max(0, np.rint(np.float32(-lo / s)))))
    q = [int(min(ASYM_QMAX, max(0, int(np.rint(np.float32(v / s))) + z))) for v in vals]
    return q, s, z


def dequantize_asym(q: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """W_hat = s * (q - z) in fp64 (exact)."""
    n, k = q.shape
    ss = np.repeat(s.astype(np.float64), GROUP, axis=1)
    zz = np.repeat(z.astype(np.float64), GROUP, axis=1)
    return (q.astype(np.float64) - zz) * ss


def encode_asym(w: np.ndarray):
    """fp32 W -> canonical (codes uint8 [n, k/2], scales fp32 [n, k/32], zeros uint8 [n, k/32])."""
    q, s, z = quantize_asym(w)
    return bitstream.pack_bits(q, 4), s, z


def algorithmic_bytes_asym(n: int, k: int) -> int:
    """16 code bytes, a 4-byte scale and a 1-byte zero point per group of 32."""
    return n * (k // GROUP) * (16 + 4 + 1)


# ---- INT4 symmetric, groups of 32 with an fp16 scale ("q4g32h") -----------------------------
#
# Source: "二三五六位量化" page, section 2.1 (each group of 32 storing its scale in fp16
# costs 16 bits per 32 weights, 0.5 bpw; the 5- and 6-bit tiers even do with a plain
# single-level group scale) and the DBHOO-CIM page, sections 2.1 and 3.1 (the INT4 rule).
#
# Readings: the INT4 rule with the scale stored as fp16: s32 = max|w| / 8 in fp32, rounded
# to the nearest fp16 (ties to even); a scale that rounds to 0 is raised to the smallest
# fp16 subnormal 2^-24 (the fp16 counterpart of the 1e-12 floor); one that overflows fp16
# is an error. The codes are then taken against the stored scale, q = clamp(rint(w / s),
# -8, 7) in fp32 with s = float(fp16 scale), so that w_hat = q * s is what was quantized
# against. 16 + 2 bytes per group (4.5 bpw); K a multiple of 64.

HALF_SCALE_FLOOR = np.float16(2.0 ** -24)


def quantize_h(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """fp32 W [n, k] (k % 64 == 0) -> (q int8 [n, k] in [-8, 7], scale fp16 [n, k/32])."""
    w = np.asarray(w)
    if w.dtype != np.float32 or w.ndim != 2:
        raise TypeError("W must be a 2-D float32 array")
    n, k = w.shape
    if k % 64:
        raise ValueError("K must be a multiple of 64")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    g = w.reshape(n, k // GROUP, GROUP)
    amax = np.abs(g).max(axis=2) if k else np.zeros((n, 0), np.float32)
    s32 = (amax / np.float32(8.0)).astype(np.float32)
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)                          # round to nearest even
    if np.any(np.isinf(s16)):
        raise OverflowError("a group scale does not fit fp16")
    s16 = np.where(s16 == 0, HALF_SCALE_FLOOR, s16).astype(np.float16)
    s = s16.astype(np.float32)
    ratio = (g / s[..., None]).astype(np.float32)
    q = np.clip(np.rint(ratio), -8, 7).astype(np.int8)
    return q.reshape(n, k), s16


def encode_h(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """fp32 W -> canonical (codes uint8 [n, k/2], scales fp16 [n, k/32])."""
    q, s = quantize_h(w)
    return pack_codes(q), s


def algorithmic_bytes_h(n: int, k: int) -> int:
    """16 code bytes and a 2-byte scale per group of 32."""
    return n * (k // GROUP) * (16 + 2)
