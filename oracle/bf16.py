"""bfloat16 helpers for the oracle: the super-scales of the "_bf16" super-block variants.

Source: "二三五六位量化" page, section 2.3 (after the byte table): an fp16 super-block scale
must cover the largest weight and can overflow to inf on badly trained layers; storing the
super-scale as bf16 trades a little precision for range. A bf16 value is the upper 16 bits
of an fp32 value; here bf16 values are carried as np.float32 arrays whose low 16 bits are
zero, and written out as their upper 16 bits, little-endian.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float(np.array(0x7F7F0000, np.uint32).view(np.float32))


def bf16_ceil(v: float) -> np.float32:
    """Smallest finite bf16 b with float(b) >= v, for finite v >= 0 (as np.float32)."""
    if not (v >= 0.0) or v == float("inf"):
        raise ValueError("bf16_ceil expects a finite non-negative value")
    return np.float32(bf16_ceil_array(np.array([v], np.float64))[0])


def bf16_ceil_array(v: np.ndarray) -> np.ndarray:
    """Elementwise bf16_ceil for a float64 array -> float32 array of bf16 values."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(~(v >= 0.0)):
        raise ValueError("bf16_ceil expects finite non-negative values")
    if np.any(v > BF16_MAX):
        raise OverflowError("value exceeds the bf16 range")
    with np.errstate(over="ignore"):
        f = v.astype(np.float32)                                   # round to nearest
        f = np.where(f.astype(np.float64) < v, np.nextafter(f, np.float32(np.inf)), f).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = np.where(u & 0xFFFF, (u & 0xFFFF0000) + 0x10000, u).astype(np.uint32)   # round the tail up
    out = u.view(np.float32)
    if not np.all(np.isfinite(out)):
        raise OverflowError("value exceeds the bf16 range")
    return out.reshape(v.shape)


def bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 values (float32 with zero low halves) -> uint16 bit patterns."""
    u = np.asarray(b, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("not a bf16 value")
    return (u >> 16).astype(np.uint16)


def bf16_to_le_bytes(b: np.ndarray) -> np.ndarray:
    """bf16 values [...] -> uint8 [..., 2] little-endian."""
    h = bf16_bits(b)
    return np.stack([(h & 0xFF).astype(np.uint8), (h >> 8).astype(np.uint8)], axis=-1)


def bf16_from_le_bytes(x: np.ndarray) -> np.ndarray:
    """uint8 [..., 2] little-endian -> bf16 values as float32 [...]."""
    x = np.asarray(x, dtype=np.uint8)
    h = x[..., 0].astype(np.uint32) | (x[..., 1].astype(np.uint32) << 8)
    return (h << 16).astype(np.uint32).view(np.float32)
