"""Pins for the bf16 super-scale variants of the super-block formats ("q2sb_bf16", "q3sb_bf16",
"q5sb_bf16", "q6sb_bf16") in oracle/superblock.py and oracle/bf16.py ("二三五六位量化" page,
section 2.3: the super-block scale stored as bf16 instead of fp16, against fp16 overflow).

Pins:
  * bf16_ceil against brute force over every finite non-negative bf16 value;
  * where the fp16 rule's d and dmin are powers of two (exact in both types) the bf16
    variant's fields and records equal the fp16 format's, except the scale bytes, which hold
    the bf16 bits of the same values;
  * section 3.4's half-step check, element by element, on random Laplace weights and on a
    block whose fp16 super-scale would overflow;
  * the element-by-element quantizer/encoder/decoder against the vectorized ones.
"""
import numpy as np
import pytest

from oracle import superblock as sb
from oracle.bf16 import bf16_bits, bf16_ceil, bf16_ceil_array, bf16_from_le_bytes, bf16_to_le_bytes
from workloads import laplace_weights

BASES = ["q2sb", "q3sb", "q5sb", "q6sb"]
FMTS = [b + "_bf16" for b in BASES]


def test_bf16_ceil_brute_force():
    allb = (np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    allb.sort()
    rng = np.random.default_rng(4)
    vals = np.concatenate([allb[::7], np.nextafter(allb[::7], np.inf), np.nextafter(allb[1::7], -np.inf),
                           10.0 ** rng.uniform(-30, 30, 4000), rng.uniform(0, 1, 2000)])
    vals = vals[vals <= allb[-1]]
    got = bf16_ceil_array(vals).astype(np.float64)
    want = allb[np.searchsorted(allb, vals, side="left")]
    assert np.array_equal(got, want)
    for v in vals[::211]:
        assert float(bf16_ceil(float(v))) == allb[np.searchsorted(allb, v, side="left")]
    b = bf16_ceil_array(np.array([1.0, 3.0e-5, 7.5e9]))
    assert np.array_equal(bf16_from_le_bytes(bf16_to_le_bytes(b)), b)
    assert bf16_bits(np.float32(1.0)) == 0x3F80


def _power_of_two_block(fmt, rng):
    """A super-block on which the fp16 rule picks power-of-two d (and dmin): the largest
    weight (and the most negative one) are placed so that T / Smax (and L / Smax) is 2^-e."""
    spec = sb.SPECS[fmt]
    w = rng.laplace(0, 0.004, 256)
    if spec.symmetric:
        w[5] = spec.smax * (spec.offset - 0.5) * 2.0 ** -9           # T / Smax = 2^-9
        w = np.clip(w, -w[5], w[5])
    else:
        L = spec.smax * 2.0 ** -10                                     # dmin = 2^-10, m = Smax
        w = np.clip(w, -L, None)
        w[3] = -L
        j = 3 // spec.sub
        hi = spec.cmax * spec.smax * 2.0 ** -7 - L                    # (hi + L) / cmax / Smax = 2^-7
        w[j * spec.sub + 1] = hi
        w = np.clip(w, None, hi)
    return w.astype(np.float32)


@pytest.mark.parametrize("base", BASES)
def test_equals_fp16_format_where_scales_are_powers_of_two(base):
    rng = np.random.default_rng(12)
    fmt = base + "_bf16"
    spec = sb.SPECS[fmt]
    w = np.stack([_power_of_two_block(base, rng) for _ in range(3)])
    f16 = sb.quantize(base, w)
    fb = sb.quantize(fmt, w)
    d = f16["d"].astype(np.float64)
    assert np.all(np.log2(d) == np.round(np.log2(d)))                 # the construction worked
    assert np.array_equal(fb["codes"], f16["codes"]) and np.array_equal(fb["sc"], f16["sc"])
    assert np.array_equal(fb["d"].astype(np.float64), d)
    r16 = sb.encode_fields(base, f16).reshape(3, -1)
    rb = sb.encode_fields(fmt, fb).reshape(3, -1)
    nd = 4 if not spec.symmetric else 2                                # d (and dmin) at the end
    assert np.array_equal(rb[:, :-nd], r16[:, :-nd])
    at = rb.shape[1] - nd
    assert np.array_equal(rb[:, at:at + 2].copy().view(np.uint16)[:, 0], bf16_bits(fb["d"][:, 0]))
    if not spec.symmetric:
        assert np.array_equal(fb["m"], f16["m"])
        assert np.array_equal(rb[:, -2:].copy().view(np.uint16)[:, 0], bf16_bits(fb["dmin"][:, 0]))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("seed", [1, 2])
def test_half_step_bound(fmt, seed):
    w = laplace_weights(32, 1024, 0.02, seed + 60, outlier_frac=0.002)
    w[0, 7] = np.float32(1.0e10)                   # d beyond fp16: fine in bf16
    with pytest.raises(OverflowError):
        sb.quantize(fmt.replace("_bf16", ""), w)
    f = sb.quantize(fmt, w)
    spec = sb.SPECS[fmt]
    assert f["codes"].max() <= spec.cmax and f["sc"].max() <= spec.smax
    w_hat = sb.dequantize_fields(fmt, f)
    step = sb.step_sizes(fmt, f)
    err = np.abs(w_hat - w.astype(np.float64))
    assert np.all(err <= step / 2 * (1 + 1e-12) + 1e-300)


@pytest.mark.parametrize("fmt", FMTS)
def test_vectorized_matches_scalar(fmt):
    spec = sb.SPECS[fmt]
    w = laplace_weights(3, 768, 0.02, 23, outlier_frac=0.01)
    w[1, 256:512] = 0.0
    w[2, 0:16] = np.abs(w[2, 0:16])
    w[2, 16:48] = -np.abs(w[2, 16:48])
    f = sb.quantize(fmt, w)
    rec = sb.encode_fields(fmt, f)
    for r in range(3):
        for s in range(3):
            fs = sb.quantize_block_scalar(spec, w[r, 256 * s:256 * s + 256])
            assert [int(c) for c in fs["codes"]] == f["codes"][r, s].tolist()
            assert [int(c) for c in fs["sc"]] == f["sc"][r, s].tolist()
            assert sb.scale_bits(spec, fs["d"]) == sb.scale_bits(spec, f["d"][r, s])
            rs = sb.encode_block_scalar(spec, fs)
            assert rs == bytes(rec[r, s])
            back = sb.decode_block_scalar(spec, rs)
            assert back["codes"] == fs["codes"]
            wh = sb.dequantize_block_scalar(spec, back)
            assert np.array_equal(np.array(wh), sb.decode(fmt, rec)[r, 256 * s:256 * s + 256])
    g = sb.decode_records(fmt, rec)
    assert np.array_equal(sb.scale_bits(spec, g["d"]), sb.scale_bits(spec, f["d"]))
