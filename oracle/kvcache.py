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
  * the scale d is the smallest fp16 >= max|x| / 127 (exact quotient), so the fp16 grid covers
    the group (the same range-covering rule as the super-block scales);
  * the code is the plain definition q = clamp(rint(x / d), -127, 127) on the exact quotient,
    rint rounding halves to even; an all-zero group has d = 0 and q = 0;
  * decode: x_hat = d * q (exact: 11 x 7 significant bits). The fp16 decode rounds it once to
    the nearest fp16 and saturates at +-65504: the one group whose d exceeds 65504 / 127 (a
    group maximum above 65469, d = 516) would otherwise decode code +-127 (+-65532) to inf.
    Saturation keeps every decoded element within d/2 of its input there, since such inputs
    are at most 65504.

Both divisions are carried out in fp64, and neither rounding can change a decision: the
operands are fp16, so a quotient that is not exactly an fp16 value (for d) or a half-integer
(for q) stays at least 2^-20 of its own size away from one (11-bit operands, quotients below
2^7), while an fp64 quotient is within 2^-53 of its size of the exact one. Exact
half-integers (x = 1.5 d, ...) come out exact and go to the even code.

Parity status: pinned by tests/test_oracle_kvcache.py (the page's byte arithmetic, hand-worked
groups in tests/golden/kvcache_groups.json, including exact ties that a reciprocal multiply
decides the other way, the d/2 error bound, saturation at the fp16 maximum, exact rational
brute force of the code decision, all-zero and one-hot groups).
"""
from __future__ import annotations

import numpy as np

from .fp16 import FP16_MAX, fp16_ceil_array

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
    g = x.astype(np.float64).reshape(rows, cols // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2)
    d = fp16_ceil_array(amax / QMAX)                                  # smallest fp16 >= max|x| / 127
    d64 = d.astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        quotient = np.where(d64 > 0, g / np.where(d64 > 0, d64, 1.0), 0.0)
    q = np.clip(np.rint(quotient), -QMAX, QMAX).astype(np.int8)      # np.rint: halves to even
    return q.reshape(rows, cols), d


def dequantize(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """(int8 codes [rows, cols], fp16 scales [rows, cols/32]) -> fp32 x_hat [rows, cols] (exact)."""
    q = np.asarray(q, dtype=np.int8)
    rows, cols = q.shape
    d32 = np.asarray(d, dtype=np.float16).astype(np.float32)
    return (q.astype(np.float32).reshape(rows, cols // GROUP, GROUP) * d32[:, :, None]).reshape(rows, cols)


def dequantize_fp16(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """The fp16 decode: d * q rounded once to the nearest fp16, saturated at +-65504."""
    v = dequantize(q, d).astype(np.float64)
    return np.clip(v, -FP16_MAX, FP16_MAX).astype(np.float16)
