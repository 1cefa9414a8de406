"""Pins for "q3sb_planes" in oracle/superblock.py: the 3-bit super-block record with its codes
split into a 2-bit plane and a 1-bit plane ("二三五六位量化" page section 2.3: widths that do not
divide a byte are stored as byte-friendly planes, as the 5- and 6-bit records are).

Pins: the same fields and W_hat as q3sb for the same weights; the code bytes are the scalar
2-bit and 1-bit streams of c & 3 and c >> 2 (bit by bit); the metadata bytes equal q3sb's;
scalar and vectorized encoders and decoders agree; record size 110 bytes.
"""
import numpy as np

from oracle import bitstream
from oracle import superblock as sb
from workloads import laplace_weights


def test_same_fields_and_w_hat_as_q3sb():
    w = laplace_weights(6, 768, 0.02, 41, outlier_frac=0.01)
    f3 = sb.quantize("q3sb", w)
    fp = sb.quantize("q3sb_planes", w)
    for key in ("codes", "sc"):
        assert np.array_equal(f3[key], fp[key])
    rec3 = sb.encode_fields("q3sb", f3)
    recp = sb.encode_fields("q3sb_planes", fp)
    assert recp.shape[-1] == 110
    assert np.array_equal(recp[..., 96:], rec3[..., 96:])          # sub-scales and d unchanged
    assert np.array_equal(sb.decode("q3sb_planes", recp), sb.decode("q3sb", rec3))


def test_plane_bytes_bit_by_bit():
    w = laplace_weights(2, 256, 0.02, 42)
    f = sb.quantize("q3sb_planes", w)
    rec = sb.encode_fields("q3sb_planes", f)
    for r in range(2):
        c = [int(v) for v in f["codes"][r, 0]]
        assert bytes(rec[r, 0, 0:64]) == bitstream.pack_bits_scalar([v & 3 for v in c], 2)
        assert bytes(rec[r, 0, 64:96]) == bitstream.pack_bits_scalar([v >> 2 for v in c], 1)
        spec = sb.SPECS["q3sb_planes"]
        fs = sb.quantize_block_scalar(spec, w[r])
        assert sb.encode_block_scalar(spec, fs) == bytes(rec[r, 0])
        back = sb.decode_block_scalar(spec, bytes(rec[r, 0]))
        assert back["codes"] == c
