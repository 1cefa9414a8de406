"""IEEE binary16 helpers for the oracle (NumPy's float16 is the primitive).

The super-block formats store their super-block scales d and dmin as fp16 ("二三五六位量化"
page, section 2.1 and the section 2.3 byte table). The quantizer needs the smallest fp16
that is >= a given fp64 value, so that the fp16 grid still covers the block (see
``superblock``); overflow is an error, as section 2.3 warns that an fp16 super-scale can
overflow to inf.
"""
from __future__ import annotations

import numpy as np

FP16_MAX = 65504.0


def fp16_ceil(v: float) -> np.float16:
    """Smallest finite fp16 h with float(h) >= v, for finite v >= 0 (subnormals allowed)."""
    if not (v >= 0.0) or v == float("inf"):
        raise ValueError("fp16_ceil expects a finite non-negative value")
    if v > FP16_MAX:
        raise OverflowError("value exceeds the fp16 range")
    h = np.float16(v)                       # round to nearest even, directly from fp64
    if float(h) < v:
        h = np.nextafter(h, np.float16(np.inf))
    if not np.isfinite(h):
        raise OverflowError("value exceeds the fp16 range")
    return np.float16(h)


def fp16_ceil_array(v: np.ndarray) -> np.ndarray:
    """Elementwise fp16_ceil for a float64 array."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(~(v >= 0.0)):
        raise ValueError("fp16_ceil expects finite non-negative values")
    if np.any(v > FP16_MAX):
        raise OverflowError("value exceeds the fp16 range")
    h = v.astype(np.float16)
    low = h.astype(np.float64) < v
    with np.errstate(over="ignore"):
        h = np.where(low, np.nextafter(h, np.float16(np.inf)), h).astype(np.float16)
    if not np.all(np.isfinite(h)):
        raise OverflowError("value exceeds the fp16 range")
    return h


def to_le_bytes(h: np.ndarray) -> np.ndarray:
    """fp16 array [...] -> uint8 [..., 2] little-endian IEEE binary16 bytes."""
    u = np.asarray(h, dtype=np.float16).view(np.uint16).astype(np.uint16)
    return np.stack([(u & 0xFF).astype(np.uint8), (u >> 8).astype(np.uint8)], axis=-1)


def from_le_bytes(b: np.ndarray) -> np.ndarray:
    """uint8 [..., 2] little-endian -> fp16 [...]."""
    b = np.asarray(b, dtype=np.uint8)
    u = b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8)
    return u.view(np.float16)
