"""Little-endian bitstreams of b-bit codes (b = 1..8).

Source: "二三五六位量化" page, section 2.2. Its ``unpack3`` assembles three bytes into a
24-bit little-endian word v = p0 | p1 << 8 | p2 << 16 and reads code i as (v >> 3i) & 7;
``unpack5`` does the same with five bytes and (v >> 5i) & 0x1F; the text says 6-bit codes
go four to three bytes the same way. (The extracted text lost the operators; the masks and
shift widths admit only this reading.) The DBHOO-CIM page, section 3.2, stores INT4 with
the first weight in the low nibble, which is the same rule at b = 4.

The general rule all of these instances follow: code i occupies stream bits
[b*i, b*i + b), least significant bit first, and stream bit j is bit (j mod 8) of byte
j div 8. A trailing partial byte is zero-padded.
"""
from __future__ import annotations

from typing import Iterable, List

import numpy as np


def packed_len(count: int, bits: int) -> int:
    return (count * bits + 7) // 8


def pack_bits_scalar(codes: Iterable[int], bits: int) -> bytes:
    """Bit-by-bit reference packer (small inputs only)."""
    codes = list(codes)
    out = bytearray(packed_len(len(codes), bits))
    for i, c in enumerate(codes):
        c = int(c)
        if not 0 <= c < (1 << bits):
            raise ValueError(f"code {c} does not fit in {bits} bits")
        for b in range(bits):
            if (c >> b) & 1:
                pos = bits * i + b
                out[pos // 8] |= 1 << (pos % 8)
    return bytes(out)


def unpack_bits_scalar(buf: bytes, bits: int, count: int) -> List[int]:
    """Bit-by-bit reference unpacker (small inputs only)."""
    if len(buf) < packed_len(count, bits):
        raise ValueError("buffer too short")
    out = []
    for i in range(count):
        c = 0
        for b in range(bits):
            pos = bits * i + b
            c |= ((buf[pos // 8] >> (pos % 8)) & 1) << b
        out.append(c)
    return out


def pack_bits(codes: np.ndarray, bits: int) -> np.ndarray:
    """Vectorized packer over the last axis: uint8 [..., count] -> uint8 [..., ceil(count*bits/8)].

    Uses NumPy's bit (un)packing with little-endian bit order as the primitive; the
    bit order of the stream is exactly the scalar packer's.
    """
    codes = np.asarray(codes)
    if codes.size and (codes.min() < 0 or codes.max() >= (1 << bits)):
        raise ValueError(f"codes do not fit in {bits} bits")
    c8 = codes.astype(np.uint8)
    bitplanes = np.unpackbits(c8[..., None], axis=-1, bitorder="little")[..., :bits]
    flat = bitplanes.reshape(*c8.shape[:-1], c8.shape[-1] * bits)
    return np.packbits(flat, axis=-1, bitorder="little")


def unpack_bits(buf: np.ndarray, bits: int, count: int) -> np.ndarray:
    """Vectorized unpacker over the last axis: uint8 [..., nbytes] -> uint8 [..., count]."""
    buf = np.asarray(buf, dtype=np.uint8)
    if buf.shape[-1] < packed_len(count, bits):
        raise ValueError("buffer too short")
    stream = np.unpackbits(buf, axis=-1, bitorder="little")[..., : count * bits]
    fields = stream.reshape(*buf.shape[:-1], count, bits).astype(np.uint16)
    weights = (1 << np.arange(bits, dtype=np.uint16))
    return (fields * weights).sum(axis=-1).astype(np.uint8)
