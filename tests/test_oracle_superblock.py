"""Pins for oracle/superblock.py and oracle/fp16.py (2/3/5/6-bit 256-weight super-blocks).

Pins:
  * the pages' byte table: 84 / 110 / 176 / 210 B per super-block = 2.625 / 3.4375 / 5.5 /
    6.5625 bpw, the 7B sizes of section 1.3 and the section 4.1 mixed-width arithmetic
    (tests/golden/sizes.json);
  * hand-worked blocks for each format (tests/golden/superblock_examples.json): fields,
    codes and selected record bytes (plane order, nibble split, 6-bit field packing, fp16
    byte order);
  * section 3.4's check: every element within half its sub-block step d*sc_j;
  * fp16_ceil against brute force over every finite binary16 value;
  * the element-by-element quantizer/encoder/decoder against the vectorized ones;
  * dequantization with all sc = 1, m = 0 reduces to textbook affine d*(c - o);
  * special cases: zero block, single-sign blocks, fp16 overflow of d.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import superblock as sb
from oracle.fp16 import fp16_ceil, fp16_ceil_array
from workloads import laplace_weights

SIZES = json.load(open(os.path.join(GOLDEN, "sizes.json")))
EXAMPLES = json.load(open(os.path.join(GOLDEN, "superblock_examples.json")))["examples"]
FMTS = ["q2sb", "q3sb", "q5sb", "q6sb"]


def _parse(v: str) -> np.float32:
    if v.startswith("fp32:"):
        return np.float32(float(v[5:]))
    num, _, den = v.partition("/")
    f = Fraction(num) / Fraction(den or "1")
    x = np.float32(float(f))
    assert Fraction(float(x)) == f, "fixture weights must be exact in fp32"
    return x


@pytest.mark.parametrize("fmt", FMTS)
def test_record_bytes_match_page_table(fmt):
    t = SIZES["superblock"][fmt]
    assert sb.SPECS[fmt].record_bytes == t["bytes"]
    w = laplace_weights(3, 512, 0.02, 11)
    rec = sb.encode(fmt, w)
    assert rec.shape == (3, 2, t["bytes"])
    assert 8 * t["bytes"] / 256 == t["bpw"]
    assert round(7e9 * t["bpw"] / 8 / 1e9, 1) == t["size_7b_gb_rounded"]
    assert sb.algorithmic_bytes(fmt, 3, 512) == rec.nbytes


def test_mixed_width_arithmetic():
    m = SIZES["mixed_7b"]
    trunk = m["trunk_params"] * SIZES["superblock"][m["trunk_fmt"]]["bpw"] / 8 / 1e9
    vocab = m["vocab_params"] * SIZES["superblock"][m["vocab_fmt"]]["bpw"] / 8 / 1e9
    assert abs(trunk - m["trunk_gb_approx"]) < 0.01 and abs(vocab - m["vocab_gb_approx"]) < 0.01
    assert abs(trunk + vocab - m["total_gb_approx"]) < 0.01


@pytest.mark.parametrize("ex", EXAMPLES, ids=lambda e: e["fmt"])
def test_hand_worked_examples(ex):
    fmt = ex["fmt"]
    spec = sb.SPECS[fmt]
    w = np.zeros(256, np.float32)
    for pos, v in ex["w"].items():
        w[int(pos)] = _parse(v)
    for f in (sb.quantize_block_scalar(spec, w),
              {k: (None if v is None else v[0, 0]) for k, v in sb.quantize(fmt, w[None, :]).items()}):
        assert int(np.float16(f["d"]).view(np.uint16)) == int(ex["d_bits"], 16)
        if ex["dmin_bits"] is None:
            assert f["dmin"] is None
        else:
            assert int(np.float16(f["dmin"]).view(np.uint16)) == int(ex["dmin_bits"], 16)
        assert [int(s) for s in f["sc"]] == ex["sc"]
        if ex["m"] is None:
            assert f["m"] is None
        else:
            assert [int(s) for s in f["m"]] == ex["m"]
        codes = [int(c) for c in f["codes"]]
        for i in range(256):
            j = i // spec.sub
            want = ex["codes"].get(str(i), ex["default_codes"].get(str(j), ex["default_codes"].get("*")))
            assert codes[i] == want, (i, codes[i], want)
    rec = sb.encode_block_scalar(spec, sb.quantize_block_scalar(spec, w))
    assert bytes(sb.encode(fmt, w[None, :])[0, 0]) == rec
    for off, hexs in ex["record_bytes"].items():
        want = bytes.fromhex(hexs.replace(" ", ""))
        assert rec[int(off):int(off) + len(want)] == want, (off, rec[int(off):int(off) + len(want)].hex())
    # section 3.4: within half a sub-block step
    f = sb.quantize_block_scalar(spec, w)
    w_hat = sb.dequantize_block_scalar(spec, f)
    for i in range(256):
        step = float(f["d"]) * f["sc"][i // spec.sub]
        assert abs(w_hat[i] - float(w[i])) <= step / 2 * (1 + 1e-12)


def test_fp16_ceil_brute_force():
    allh = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)   # all finite >= 0
    allh.sort()
    rng = np.random.default_rng(3)
    vals = np.concatenate([allh, np.nextafter(allh, np.inf), np.nextafter(allh, -np.inf)[1:],
                           rng.uniform(0, 65504, 2000), 10.0 ** rng.uniform(-9, 4.8, 4000)])
    vals = vals[(vals >= 0) & (vals <= 65504)]
    got = fp16_ceil_array(vals).astype(np.float64)
    want = allh[np.searchsorted(allh, vals, side="left")]
    assert np.array_equal(got, want)
    for v in vals[::97]:
        assert float(fp16_ceil(float(v))) == allh[np.searchsorted(allh, v, side="left")]
    with pytest.raises(OverflowError):
        fp16_ceil(65504.5)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("seed", [1, 2])
def test_half_step_bound_random(fmt, seed):
    w = laplace_weights(32, 1024, 0.02, seed + 40, outlier_frac=0.002)
    f = sb.quantize(fmt, w)
    spec = sb.SPECS[fmt]
    assert f["codes"].max() <= spec.cmax
    assert f["sc"].min() >= 0 and f["sc"].max() <= spec.smax
    if f["m"] is not None:
        assert f["m"].min() >= 0 and f["m"].max() <= spec.smax
    assert np.all(np.isfinite(f["d"].astype(np.float64)))
    w_hat = sb.dequantize_fields(fmt, f)
    step = sb.step_sizes(fmt, f)
    err = np.abs(w_hat - w.astype(np.float64))
    assert np.all(err <= step / 2 * (1 + 1e-12) + 1e-300)


@pytest.mark.parametrize("fmt", FMTS)
def test_vectorized_matches_scalar(fmt):
    spec = sb.SPECS[fmt]
    w = laplace_weights(4, 768, 0.02, 21, outlier_frac=0.01)
    w[1, 256:512] = 0.0                      # a zero super-block
    w[2, 0:16] = np.abs(w[2, 0:16])          # positive-only sub-block
    w[2, 16:48] = -np.abs(w[2, 16:48])       # negative-only sub-blocks
    w[3, 512:768] = np.float32(0.01)         # constant super-block
    f = sb.quantize(fmt, w)
    rec = sb.encode_fields(fmt, f)
    for r in range(4):
        for s in range(3):
            fs = sb.quantize_block_scalar(spec, w[r, 256 * s:256 * s + 256])
            assert [int(c) for c in fs["codes"]] == f["codes"][r, s].tolist()
            assert [int(c) for c in fs["sc"]] == f["sc"][r, s].tolist()
            assert np.float16(fs["d"]).view(np.uint16) == f["d"][r, s].view(np.uint16)
            rs = sb.encode_block_scalar(spec, fs)
            assert rs == bytes(rec[r, s])
            back = sb.decode_block_scalar(spec, rs)
            assert back["codes"] == fs["codes"] and list(back["sc"]) == list(fs["sc"])
            wh = sb.dequantize_block_scalar(spec, back)
            assert np.array_equal(np.array(wh), sb.decode(fmt, rec)[r, 256 * s:256 * s + 256])


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_inverts_encode(fmt):
    w = laplace_weights(8, 512, 0.02, 31)
    f = sb.quantize(fmt, w)
    g = sb.decode_records(fmt, sb.encode_fields(fmt, f))
    for key in ("codes", "sc", "m"):
        if f[key] is None:
            assert g[key] is None
        else:
            assert np.array_equal(f[key], g[key])
    assert np.array_equal(f["d"].view(np.uint16), g["d"].view(np.uint16))


@pytest.mark.parametrize("fmt", FMTS)
def test_affine_special_case(fmt):
    """With every sub-scale 1 and every min 0 the format is textbook affine: d * (c - o)."""
    spec = sb.SPECS[fmt]
    rng = np.random.default_rng(5)
    codes = rng.integers(0, spec.cmax + 1, size=(2, 1, 256)).astype(np.uint8)
    d = np.array([[0.5], [0.0078125]], np.float16)
    f = dict(codes=codes, sc=np.ones((2, 1, spec.nsub), np.int16),
             m=None if spec.symmetric else np.zeros((2, 1, spec.nsub), np.int16),
             d=d, dmin=None if spec.symmetric else np.zeros((2, 1), np.float16))
    w_hat = sb.dequantize_fields(fmt, f)
    want = d.astype(np.float64) * (codes[:, 0, :].astype(np.float64) - spec.offset)
    assert np.array_equal(w_hat, want)
    rec = sb.encode_fields(fmt, f)
    assert np.array_equal(sb.decode(fmt, rec), want)


@pytest.mark.parametrize("fmt", FMTS)
def test_zero_block_and_overflow(fmt):
    w = np.zeros((1, 256), np.float32)
    f = sb.quantize(fmt, w)
    assert float(f["d"][0, 0]) == 0.0 and np.all(sb.dequantize_fields(fmt, f) == 0.0)
    big = np.zeros((1, 256), np.float32)
    big[0, 0] = 1.0e10                        # needs d > 65504
    with pytest.raises(OverflowError):
        sb.quantize(fmt, big)
    bad = np.zeros((1, 256), np.float32)
    bad[0, 7] = np.inf
    with pytest.raises(ValueError):
        sb.quantize(fmt, bad)
