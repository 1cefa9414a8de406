"""256-weight super-block formats at 2, 3, 5 and 6 bits ("q2sb", "q3sb", "q5sb", "q6sb").

Source: "二三五六位量化" page.
  * Section 2.1: three-tier scales: an fp16 super-block scale, low-bit sub-block scales,
    then the codes, over a 256-weight super-block; 5- and 6-bit need only group 32.
  * Section 2.2: little-endian cross-byte packing (3-bit: 8 codes in 3 bytes; 5-bit: 8
    in 5; 6-bit: 4 in 3).
  * Section 2.3 byte table (per 256 weights):
        2-bit: 64 B codes + 16 sub-blocks x 8 bit (16 B) + fp16 d and dmin (4 B) =  84 B
        3-bit: 96 B codes + 16 x 6-bit sub-scales packed (12 B) + fp16 d (2 B)   = 110 B
        5-bit: 128 B low-4-bit plane + 32 B high-1-bit plane + 12 B + d, dmin  = 176 B
        6-bit: 128 B low-4-bit plane + 64 B high-2-bit plane + 16 B int8 + d     = 210 B
    and the text after it: 16 sub-blocks of 16 weights at 2 and 3 bits; 5- and 6-bit codes
    are split into a low-4-bit plane plus a high-bit plane.
  * Section 3.3: the scalar GEMV form acc += (s*q + m) * x, and its rewrite
    s*(q.x) + m*sum(x).
  * Section 3.4: self-checks (round trip; single-group dequant error below half a step).

Readings (the pages give the layouts but not every field, nor how scales are chosen):
  * Sub-block counts follow from the byte counts: q2sb 16 x 16 (8 bits each = 4-bit scale
    in the low nibble, 4-bit min in the high nibble); q3sb 16 x 16 (12 B = 16 x 6 bit);
    q5sb 8 x 32 (12 B = 8 six-bit scales then 8 six-bit mins, section 2.1's "group 32"
    for 5/6-bit); q6sb 16 x 16 (16 B = 16 int8 scales).
  * Two records carry a dmin (2- and 5-bit): those are asymmetric,
        w_hat = d * sc_j * c - dmin * m_j,   c in [0, 2^b - 1].
    The other two (3- and 6-bit) carry only d: symmetric with a fixed code offset o,
        w_hat = d * sc_j * (c - o),  o = 4 (3-bit) or 32 (6-bit).
    (Section 2.1's remark that low bit widths "must be asymmetric" contradicts its own
    3-bit record, which has no dmin; the record wins.)
  * Every packed field is a little-endian bitstream (bitstream.py). Record field order is
    the table's column order: codes [, high plane], sub-scales, d [, dmin]. A 5/6-bit code
    is c = low4 | high << 4.
  * q6sb sub-scales are decoded as signed int8 (the table says int8); this quantizer only
    produces 0..127.
  * Scale choice ("range-covering round to nearest"), in fp64, with fp16_ceil = smallest
    fp16 >= v:
      symmetric (b, o, Smax): t_j = max|w_j| / (o - 0.5); T = max_j t_j;
          d = fp16_ceil(T / Smax); sc_j = min(Smax, ceil(t_j / d));
          c = clamp(rint(w / (d * sc_j)) + o, 0, 2^b - 1)
      asymmetric (b, Smax): lo_j = min(0, min w_j), hi_j = max(0, max w_j);
          dmin = fp16_ceil(max_j(-lo_j) / Smax); m_j = min(Smax, ceil(-lo_j / dmin));
          off_j = dmin * m_j; t_j = (hi_j + off_j) / (2^b - 1);
          d = fp16_ceil(max_j t_j / Smax); sc_j = min(Smax, ceil(t_j / d));
          c = clamp(rint((w + off_j) / (d * sc_j)), 0, 2^b - 1)
    A zero maximum gives d = 0 (dmin = 0), sc = 0 (m = 0) and c = o (c = 0). This keeps
    |w - w_hat| <= d * sc_j / 2 for every element, which is section 3.4's check with
    "scale" read as the sub-block step d * sc_j. rint is round half to even.
  * A super-scale beyond the fp16 range raises OverflowError (section 2.3 warns of inf).
  * "q3sb_planes": section 2.3's advice for widths that do not divide a byte (split the code
    into byte-friendly planes instead of interleaving, as the 5- and 6-bit records do) applied
    to the 3-bit record: the same fields and rule as q3sb, with the 96 code bytes stored as a
    64-byte plane of the low 2 bits (2-bit little-endian stream) followed by a 32-byte plane
    of the high bit (1-bit stream); 110 bytes as before.
  * bf16 super-scales ("q2sb_bf16", "q3sb_bf16", "q5sb_bf16", "q6sb_bf16"): section 2.3's
    remedy for that overflow, storing the super-block scale as bf16. Read as the same
    format, record layout and rule with bf16_ceil (smallest bf16 >= v) in place of
    fp16_ceil for d and dmin, and the two bytes of each holding the bf16 bits.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List

import numpy as np

from . import bitstream
from .bf16 import bf16_bits, bf16_ceil, bf16_ceil_array, bf16_from_le_bytes, bf16_to_le_bytes
from .fp16 import fp16_ceil, fp16_ceil_array, from_le_bytes, to_le_bytes

QK = 256


@dataclasses.dataclass(frozen=True)
class SBSpec:
    name: str
    bits: int
    nsub: int
    symmetric: bool
    offset: int
    smax: int
    record_bytes: int
    layout: str = ""           # the base format whose record layout this one shares
    bf16: bool = False         # super-scales d, dmin stored as bf16 instead of fp16

    @property
    def sub(self) -> int:
        return QK // self.nsub

    @property
    def cmax(self) -> int:
        return (1 << self.bits) - 1


SPECS: Dict[str, SBSpec] = {
    "q2sb": SBSpec("q2sb", 2, 16, False, 0, 15, 84, "q2sb"),
    "q3sb": SBSpec("q3sb", 3, 16, True, 4, 63, 110, "q3sb"),
    "q5sb": SBSpec("q5sb", 5, 8, False, 0, 63, 176, "q5sb"),
    "q6sb": SBSpec("q6sb", 6, 16, True, 32, 127, 210, "q6sb"),
}
for _b in ("q2sb", "q3sb", "q5sb", "q6sb"):
    SPECS[_b + "_bf16"] = dataclasses.replace(SPECS[_b], name=_b + "_bf16", bf16=True)
SPECS["q3sb_planes"] = dataclasses.replace(SPECS["q3sb"], name="q3sb_planes", layout="q3sb_planes")


# Super-scale codec of a spec: ceil to the stored type, zero, bits, little-endian bytes.
def _ceil(spec: SBSpec, v: float):
    return bf16_ceil(v) if spec.bf16 else fp16_ceil(v)


def _ceil_array(spec: SBSpec, v: np.ndarray) -> np.ndarray:
    return bf16_ceil_array(v) if spec.bf16 else fp16_ceil_array(v)


def _zero(spec: SBSpec):
    return np.float32(0.0) if spec.bf16 else np.float16(0.0)


def _dtype(spec: SBSpec):
    return np.float32 if spec.bf16 else np.float16


def scale_bits(spec: SBSpec, d) -> np.ndarray:
    """Stored 16-bit pattern of super-scales (fp16 or bf16 per spec)."""
    d = np.asarray(d, _dtype(spec))
    return bf16_bits(d) if spec.bf16 else d.view(np.uint16)


def _to_bytes(spec: SBSpec, d) -> np.ndarray:
    return bf16_to_le_bytes(d) if spec.bf16 else to_le_bytes(d)


def _from_bytes(spec: SBSpec, b) -> np.ndarray:
    return bf16_from_le_bytes(b) if spec.bf16 else from_le_bytes(b)


# ---------------------------------------------------------------------------
# One super-block, element by element (the reference form)
# ---------------------------------------------------------------------------

def quantize_block_scalar(spec: SBSpec, w256) -> dict:
    vals = [float(np.float32(v)) for v in w256]
    if len(vals) != QK:
        raise ValueError("a super-block has 256 weights")
    if not all(math.isfinite(v) for v in vals):
        raise ValueError("non-finite weight")
    sub, nsub, cmax = spec.sub, spec.nsub, spec.cmax
    blocks = [vals[j * sub:(j + 1) * sub] for j in range(nsub)]
    codes: List[int] = []
    if spec.symmetric:
        o = spec.offset
        t = [max(abs(v) for v in blk) / (o - 0.5) for blk in blocks]
        T = max(t)
        if T == 0.0:
            return dict(codes=[o] * QK, sc=[0] * nsub, m=None, d=_zero(spec), dmin=None)
        d = _ceil(spec, T / spec.smax)
        dd = float(d)
        sc = [min(spec.smax, math.ceil(tj / dd)) for tj in t]
        for j, blk in enumerate(blocks):
            step = dd * sc[j]
            for v in blk:
                codes.append(o if step == 0.0 else min(cmax, max(0, round(v / step) + o)))
        return dict(codes=codes, sc=sc, m=None, d=d, dmin=None)
    lo = [min(0.0, min(blk)) for blk in blocks]
    hi = [max(0.0, max(blk)) for blk in blocks]
    L = max(-x for x in lo)
    if L == 0.0:
        dmin = _zero(spec)
        m = [0] * nsub
    else:
        dmin = _ceil(spec, L / spec.smax)
        m = [min(spec.smax, math.ceil(-x / float(dmin))) for x in lo]
    off = [float(dmin) * mj for mj in m]
    t = [(hi[j] + off[j]) / cmax for j in range(nsub)]
    T = max(t)
    if T == 0.0:
        d = _zero(spec)
        sc = [0] * nsub
    else:
        d = _ceil(spec, T / spec.smax)
        sc = [min(spec.smax, math.ceil(tj / float(d))) for tj in t]
    for j, blk in enumerate(blocks):
        step = float(d) * sc[j]
        for v in blk:
            codes.append(0 if step == 0.0 else min(cmax, max(0, round((v + off[j]) / step))))
    return dict(codes=codes, sc=sc, m=m, d=d, dmin=dmin)


def dequantize_block_scalar(spec: SBSpec, f: dict) -> List[float]:
    out = []
    d = float(f["d"])
    for i, c in enumerate(f["codes"]):
        j = i // spec.sub
        if spec.symmetric:
            out.append(d * f["sc"][j] * (c - spec.offset))
        else:
            out.append(d * f["sc"][j] * c - float(f["dmin"]) * f["m"][j])
    return out


def encode_block_scalar(spec: SBSpec, f: dict) -> bytes:
    codes = f["codes"]
    d = _to_bytes(spec, np.array(f["d"], _dtype(spec))).tobytes()
    if spec.layout == "q2sb":
        meta = bytes((f["sc"][j] | (f["m"][j] << 4)) for j in range(16))
        dm = _to_bytes(spec, np.array(f["dmin"], _dtype(spec))).tobytes()
        rec = bitstream.pack_bits_scalar(codes, 2) + meta + d + dm
    elif spec.layout == "q3sb":
        rec = bitstream.pack_bits_scalar(codes, 3) + bitstream.pack_bits_scalar(f["sc"], 6) + d
    elif spec.layout == "q3sb_planes":
        rec = (bitstream.pack_bits_scalar([c & 3 for c in codes], 2)
               + bitstream.pack_bits_scalar([c >> 2 for c in codes], 1)
               + bitstream.pack_bits_scalar(f["sc"], 6) + d)
    elif spec.layout == "q5sb":
        dm = _to_bytes(spec, np.array(f["dmin"], _dtype(spec))).tobytes()
        rec = (bitstream.pack_bits_scalar([c & 15 for c in codes], 4)
               + bitstream.pack_bits_scalar([c >> 4 for c in codes], 1)
               + bitstream.pack_bits_scalar(list(f["sc"]) + list(f["m"]), 6) + d + dm)
    elif spec.layout == "q6sb":
        rec = (bitstream.pack_bits_scalar([c & 15 for c in codes], 4)
               + bitstream.pack_bits_scalar([c >> 4 for c in codes], 2)
               + bytes((s & 0xFF) for s in f["sc"]) + d)
    else:
        raise KeyError(spec.name)
    assert len(rec) == spec.record_bytes
    return rec


def decode_block_scalar(spec: SBSpec, rec: bytes) -> dict:
    if len(rec) != spec.record_bytes:
        raise ValueError("wrong record length")

    def half(b):
        return _from_bytes(spec, np.frombuffer(b, np.uint8)).reshape(())[()]

    if spec.layout == "q2sb":
        codes = bitstream.unpack_bits_scalar(rec[0:64], 2, QK)
        sc = [b & 15 for b in rec[64:80]]
        m = [b >> 4 for b in rec[64:80]]
        return dict(codes=codes, sc=sc, m=m, d=half(rec[80:82]), dmin=half(rec[82:84]))
    if spec.layout == "q3sb_planes":
        lo = bitstream.unpack_bits_scalar(rec[0:64], 2, QK)
        hi = bitstream.unpack_bits_scalar(rec[64:96], 1, QK)
        sc = bitstream.unpack_bits_scalar(rec[96:108], 6, 16)
        return dict(codes=[a | (b << 2) for a, b in zip(lo, hi)], sc=sc, m=None, d=half(rec[108:110]), dmin=None)
    if spec.layout == "q3sb":
        codes = bitstream.unpack_bits_scalar(rec[0:96], 3, QK)
        sc = bitstream.unpack_bits_scalar(rec[96:108], 6, 16)
        return dict(codes=codes, sc=sc, m=None, d=half(rec[108:110]), dmin=None)
    if spec.layout == "q5sb":
        lo = bitstream.unpack_bits_scalar(rec[0:128], 4, QK)
        hi = bitstream.unpack_bits_scalar(rec[128:160], 1, QK)
        f6 = bitstream.unpack_bits_scalar(rec[160:172], 6, 16)
        return dict(codes=[a | (b << 4) for a, b in zip(lo, hi)], sc=f6[:8], m=f6[8:],
                    d=half(rec[172:174]), dmin=half(rec[174:176]))
    if spec.layout == "q6sb":
        lo = bitstream.unpack_bits_scalar(rec[0:128], 4, QK)
        hi = bitstream.unpack_bits_scalar(rec[128:192], 2, QK)
        sc = [b - 256 if b >= 128 else b for b in rec[192:208]]
        return dict(codes=[a | (b << 4) for a, b in zip(lo, hi)], sc=sc, m=None, d=half(rec[208:210]), dmin=None)
    raise KeyError(spec.name)


# ---------------------------------------------------------------------------
# Whole matrices, vectorized over super-blocks (same arithmetic, same order)
# ---------------------------------------------------------------------------

def quantize(fmt: str, w: np.ndarray) -> dict:
    """fp32 W [n, k] -> fields: codes uint8 [n, S, 256], sc int16 [n, S, nsub],
    m int16 [n, S, nsub] or None, d fp16 [n, S], dmin fp16 [n, S] or None."""
    spec = SPECS[fmt]
    w = np.asarray(w)
    if w.dtype != np.float32 or w.ndim != 2:
        raise TypeError("W must be a 2-D float32 array")
    n, k = w.shape
    if k % QK:
        raise ValueError("K must be a multiple of 256")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    S = k // QK
    v = w.astype(np.float64).reshape(n, S, spec.nsub, spec.sub)
    cmax = spec.cmax
    if spec.symmetric:
        o = spec.offset
        t = np.abs(v).max(axis=3) / (o - 0.5) if v.size else np.zeros((n, S, spec.nsub))
        T = t.max(axis=2) if t.size else np.zeros((n, S))
        d = _ceil_array(spec, T / spec.smax)
        d = np.where(T == 0.0, _zero(spec), d).astype(_dtype(spec))
        dd = d.astype(np.float64)[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            sc = np.minimum(spec.smax, np.ceil(t / dd))
        sc = np.where(dd == 0.0, 0.0, sc)
        step = (dd * sc)[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            c = np.clip(np.rint(v / step) + o, 0, cmax)
        c = np.where(step == 0.0, o, c)
        return dict(codes=c.reshape(n, S, QK).astype(np.uint8), sc=sc.astype(np.int16), m=None, d=d, dmin=None)
    lo = np.minimum(0.0, v.min(axis=3)) if v.size else np.zeros((n, S, spec.nsub))
    hi = np.maximum(0.0, v.max(axis=3)) if v.size else np.zeros((n, S, spec.nsub))
    L = (-lo).max(axis=2) if lo.size else np.zeros((n, S))
    dmin = _ceil_array(spec, L / spec.smax)
    dmin = np.where(L == 0.0, _zero(spec), dmin).astype(_dtype(spec))
    dm = dmin.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        m = np.minimum(spec.smax, np.ceil(-lo / dm))
    m = np.where(dm == 0.0, 0.0, m)
    off = dm * m
    t = (hi + off) / cmax
    T = t.max(axis=2) if t.size else np.zeros((n, S))
    d = _ceil_array(spec, T / spec.smax)
    d = np.where(T == 0.0, _zero(spec), d).astype(_dtype(spec))
    dd = d.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.minimum(spec.smax, np.ceil(t / dd))
    sc = np.where(dd == 0.0, 0.0, sc)
    step = (dd * sc)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.clip(np.rint((v + off[..., None]) / step), 0, cmax)
    c = np.where(step == 0.0, 0, c)
    return dict(codes=c.reshape(n, S, QK).astype(np.uint8), sc=sc.astype(np.int16), m=m.astype(np.int16),
                d=d, dmin=dmin)


def encode_fields(fmt: str, f: dict) -> np.ndarray:
    """fields -> canonical records uint8 [n, S, record_bytes]."""
    spec = SPECS[fmt]
    codes = f["codes"]
    n, S, _ = codes.shape
    d = _to_bytes(spec, f["d"])
    lay = spec.layout
    if lay == "q2sb":
        meta = (f["sc"].astype(np.uint8) | (f["m"].astype(np.uint8) << 4)).astype(np.uint8)
        parts = [bitstream.pack_bits(codes, 2), meta, d, _to_bytes(spec, f["dmin"])]
    elif lay == "q3sb":
        parts = [bitstream.pack_bits(codes, 3), bitstream.pack_bits(f["sc"].astype(np.uint8), 6), d]
    elif lay == "q3sb_planes":
        parts = [bitstream.pack_bits(codes & 3, 2), bitstream.pack_bits(codes >> 2, 1),
                 bitstream.pack_bits(f["sc"].astype(np.uint8), 6), d]
    elif lay == "q5sb":
        f6 = np.concatenate([f["sc"], f["m"]], axis=-1).astype(np.uint8)
        parts = [bitstream.pack_bits(codes & 15, 4), bitstream.pack_bits(codes >> 4, 1),
                 bitstream.pack_bits(f6, 6), d, _to_bytes(spec, f["dmin"])]
    elif lay == "q6sb":
        parts = [bitstream.pack_bits(codes & 15, 4), bitstream.pack_bits(codes >> 4, 2),
                 (f["sc"].astype(np.int16) & 0xFF).astype(np.uint8), d]
    else:
        raise KeyError(fmt)
    rec = np.concatenate(parts, axis=-1)
    assert rec.shape == (n, S, spec.record_bytes)
    return rec


def decode_records(fmt: str, rec: np.ndarray) -> dict:
    """canonical records uint8 [n, S, record_bytes] -> fields."""
    spec = SPECS[fmt]
    rec = np.asarray(rec, np.uint8)
    if rec.shape[-1] != spec.record_bytes:
        raise ValueError("wrong record length")
    lay = spec.layout

    def half(b):
        return _from_bytes(spec, b)

    if lay == "q2sb":
        codes = bitstream.unpack_bits(rec[..., 0:64], 2, QK)
        meta = rec[..., 64:80]
        return dict(codes=codes, sc=(meta & 15).astype(np.int16), m=(meta >> 4).astype(np.int16),
                    d=half(rec[..., 80:82]), dmin=half(rec[..., 82:84]))
    if lay == "q3sb_planes":
        lo = bitstream.unpack_bits(rec[..., 0:64], 2, QK)
        hi = bitstream.unpack_bits(rec[..., 64:96], 1, QK)
        return dict(codes=(lo | (hi << 2)).astype(np.uint8),
                    sc=bitstream.unpack_bits(rec[..., 96:108], 6, 16).astype(np.int16), m=None,
                    d=half(rec[..., 108:110]), dmin=None)
    if lay == "q3sb":
        return dict(codes=bitstream.unpack_bits(rec[..., 0:96], 3, QK),
                    sc=bitstream.unpack_bits(rec[..., 96:108], 6, 16).astype(np.int16), m=None,
                    d=half(rec[..., 108:110]), dmin=None)
    if lay == "q5sb":
        lo = bitstream.unpack_bits(rec[..., 0:128], 4, QK)
        hi = bitstream.unpack_bits(rec[..., 128:160], 1, QK)
        f6 = bitstream.unpack_bits(rec[..., 160:172], 6, 16).astype(np.int16)
        return dict(codes=(lo | (hi << 4)).astype(np.uint8), sc=f6[..., :8], m=f6[..., 8:],
                    d=half(rec[..., 172:174]), dmin=half(rec[..., 174:176]))
    if lay == "q6sb":
        lo = bitstream.unpack_bits(rec[..., 0:128], 4, QK)
        hi = bitstream.unpack_bits(rec[..., 128:192], 2, QK)
        return dict(codes=(lo | (hi << 4)).astype(np.uint8), sc=rec[..., 192:208].view(np.int8).astype(np.int16),
                    m=None, d=half(rec[..., 208:210]), dmin=None)
    raise KeyError(fmt)


def dequantize_fields(fmt: str, f: dict) -> np.ndarray:
    """fields -> W_hat fp64 [n, k] (exact for these value ranges)."""
    spec = SPECS[fmt]
    codes = f["codes"].astype(np.float64)
    n, S, _ = codes.shape
    c = codes.reshape(n, S, spec.nsub, spec.sub)
    d = f["d"].astype(np.float64)[..., None, None]
    sc = f["sc"].astype(np.float64)[..., None]
    if spec.symmetric:
        w = d * sc * (c - spec.offset)
    else:
        dmin = f["dmin"].astype(np.float64)[..., None, None]
        m = f["m"].astype(np.float64)[..., None]
        w = d * sc * c - dmin * m
    return w.reshape(n, S * QK)


def encode(fmt: str, w: np.ndarray) -> np.ndarray:
    """fp32 W [n, k] -> canonical records uint8 [n, k/256, record_bytes]."""
    return encode_fields(fmt, quantize(fmt, w))


def decode(fmt: str, rec: np.ndarray) -> np.ndarray:
    """canonical records -> W_hat fp64 [n, k]."""
    return dequantize_fields(fmt, decode_records(fmt, rec))


def step_sizes(fmt: str, f: dict) -> np.ndarray:
    """Per-element sub-block step d * sc_j, fp64 [n, k] (the 'scale' of the half-step check)."""
    spec = SPECS[fmt]
    n, S, _ = f["codes"].shape
    st = f["d"].astype(np.float64)[..., None] * f["sc"].astype(np.float64)
    return np.repeat(st, spec.sub, axis=-1).reshape(n, S * QK)


def algorithmic_bytes(fmt: str, n: int, k: int) -> int:
    return n * (k // QK) * SPECS[fmt].record_bytes
