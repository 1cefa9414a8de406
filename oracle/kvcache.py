"""8-bit KV-cache group codec, by definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "二三五六位量化" page, section 4.1: the KV cache takes
2 x n_layer x n_kv_head x head_dim x ctx_len x bytes_per_element bytes (7B example: 32 layers,
8 KV heads, head_dim 128, 8192 tokens in fp16 = 1.07 GB); quantizing it to 8 bits with one
fp16 scale shared by every 32 elements costs about 1.06 bytes per element (8 + 16/32 bits =
8.5 bits) and halves it, with negligible loss.

Readings (the page gives the group size, the code width and the scale type only):
  * symmetric int8 codes in [-127, 127] (no zero point: K and V entries are centred, and the
    page mentions only a scale); groups are 32 consecutive elements of a row;
  * the scale d is the smallest fp16 >= max|x| / 127, so the fp16 grid covers the group and
    every element is within d/2 of its decoded value (the same range-covering rule as the
    super-block scales);
  * the code decision is made in fp32, the precision a GPU kernel computes it in (the page
    fixes none): t = fp32(max|x|) / 127 (one fp32 division), d = fp16_ceil(t),
    inv = fp32(1 / d) (one fp32 division per group), q = clamp(rint(fp32(x) * inv), -127, 127)
    with rint half-to-even; an all-zero group has d = 0, inv = 0 and q = 0. (A multiply by
    the group's reciprocal rather than a division per element: it can move a code by one only
    where x / d lies within an ulp of a half-integer, and keeps the error within d/2 up to
    that ulp.)
  * decode: x_hat = fp32(d) * q (exact in fp32: 11 x 7 significant bits), rounded once to
    fp16 for the fp16 output.

Parity status: pinned by tests/test_oracle_kvcache.py (the page's byte arithmetic, hand-worked
groups in tests/golden/kvcache_groups.json, the d/2 error bound, all-zero and one-hot groups).
"""
from __future__ import annotations

import numpy as np

from .fp16 import fp16_ceil_array

GROUP = 32
QMAX = 127


def bytes_per_element() -> float:
    """int8 code plus 2/32 bytes of fp16 scale."""
    return 1.0 + 2.0 / GROUP


def kv_cache_elements(n_layer: int, n_kv_head: int, head_dim: int, ctx_len: int) -> int:
    """K and V entries of a full cache (the factor 2 is one K and one V)."""
    return 2 * n_layer * n_kv_head * head_dim * ctx_len


def quantize(x: np.ndarray):
    """fp16 [rows, cols] (cols % 32 == 0) -> (int8 codes [rows, cols], fp16 scales [rows, cols/32])."""
    x = np.asarray(x, dtype=np.float16)
    rows, cols = x.shape
    if cols % GROUP:
        raise ValueError("cols must be a multiple of 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    g = x.astype(np.float32).reshape(rows, cols // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2)                                  # exact (fp16 values)
    t = (amax / np.float32(QMAX)).astype(np.float32)                  # one fp32 division
    d = fp16_ceil_array(t.astype(np.float64))                         # smallest fp16 >= t
    d32 = d.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore"):
        inv = np.where(d32 > 0, np.float32(1) / np.where(d32 > 0, d32, np.float32(1)), np.float32(0)).astype(np.float32)
    r = (g * inv).astype(np.float32)                                  # one fp32 multiply
    q = np.clip(np.rint(r), -QMAX, QMAX).astype(np.int8)
    return q.reshape(rows, cols), d


def dequantize(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """(int8 codes [rows, cols], fp16 scales [rows, cols/32]) -> fp32 x_hat [rows, cols] (exact)."""
    q = np.asarray(q, dtype=np.int8)
    rows, cols = q.shape
    d32 = np.asarray(d, dtype=np.float16).astype(np.float32)
    return (q.astype(np.float32).reshape(rows, cols // GROUP, GROUP) * d32[:, :, None]).reshape(rows, cols)
