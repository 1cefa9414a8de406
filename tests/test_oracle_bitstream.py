"""Pins for oracle/bitstream.py (little-endian b-bit code streams).

Pins: golden vectors hand-derived from the printed unpack3/unpack5 semantics and the INT4
low-nibble-first rule (tests/golden/bitstream.json); the pages' own self-check, a pack ->
unpack round trip on 10^6 random codes ("二三五六位量化" page, sections 2.2 and 3.4); and
the vectorized packer against the bit-by-bit one.
"""
import json
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import bitstream
from workloads import uniform_codes

VECTORS = json.load(open(os.path.join(GOLDEN, "bitstream.json")))["vectors"]


@pytest.mark.parametrize("vec", VECTORS, ids=lambda v: f"b{v['bits']}-{v['codes']}")
def test_golden_vectors(vec):
    want = bytes.fromhex(vec["bytes"].replace(" ", ""))
    assert bitstream.pack_bits_scalar(vec["codes"], vec["bits"]) == want
    assert bytes(bitstream.pack_bits(np.array(vec["codes"], np.uint8), vec["bits"])) == want
    assert bitstream.unpack_bits_scalar(want, vec["bits"], len(vec["codes"])) == vec["codes"]
    got = bitstream.unpack_bits(np.frombuffer(want, np.uint8), vec["bits"], len(vec["codes"]))
    assert got.tolist() == vec["codes"]


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6])
def test_round_trip_million(bits):
    codes = uniform_codes(1_000_000, bits, seed=1000 + bits)
    packed = bitstream.pack_bits(codes, bits)
    assert packed.shape == (bitstream.packed_len(1_000_000, bits),)
    assert np.array_equal(bitstream.unpack_bits(packed, bits, 1_000_000), codes)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6])
def test_vectorized_matches_scalar(bits):
    for count in (1, 7, 8, 9, 33, 256):
        codes = uniform_codes(count, bits, seed=77 * bits + count)
        a = bitstream.pack_bits_scalar(codes.tolist(), bits)
        b = bytes(bitstream.pack_bits(codes, bits))
        assert a == b
        assert bitstream.unpack_bits_scalar(a, bits, count) == codes.tolist()


def test_batched_rows_are_independent():
    codes = uniform_codes(5 * 256, 3, seed=5).reshape(5, 256)
    packed = bitstream.pack_bits(codes, 3)
    assert packed.shape == (5, 96)
    for r in range(5):
        assert bytes(packed[r]) == bitstream.pack_bits_scalar(codes[r].tolist(), 3)


def test_rejects_out_of_range():
    with pytest.raises(ValueError):
        bitstream.pack_bits_scalar([8], 3)
    with pytest.raises(ValueError):
        bitstream.pack_bits(np.array([64], np.uint8), 6)
