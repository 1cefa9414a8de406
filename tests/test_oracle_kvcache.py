"""Pins for oracle/kvcache.py (8-bit KV-cache groups: "二三五六位量化" page, section 4.1)."""
import json
import os
from fractions import Fraction

import numpy as np

from oracle import kvcache

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kvcache_groups.json")


def _golden_group(grp):
    x = np.zeros((1, 32), np.float16)
    for i, v in grp["values"].items():
        x[0, int(i)] = v
    return x


def test_page_byte_arithmetic():
    g = json.load(open(GOLDEN))["sizes"]
    n = kvcache.kv_cache_elements(32, 8, 128, 8192)
    assert n == g["elements"]
    assert n * 2 == g["fp16_bytes"]                   # the page's 1.07 GB
    assert n * kvcache.bytes_per_element() == g["int8_bytes"]
    assert abs(kvcache.bytes_per_element() - 1.06) < 0.005   # the page's "about 1.06"


def test_hand_worked_groups():
    for grp in json.load(open(GOLDEN))["groups"]:
        x = _golden_group(grp)
        q, d = kvcache.quantize(x)
        assert d[0, 0].view(np.uint16) == int(grp["scale_bits"], 16), (grp, hex(d[0, 0].view(np.uint16)))
        want = np.zeros(32, np.int8)
        for i, c in grp["codes"].items():
            want[int(i)] = c
        assert np.array_equal(q[0], want), (q[0], want)
        for i, bits in grp.get("fp16_decode_bits", {}).items():
            assert kvcache.dequantize_fp16(q, d)[0, int(i)].view(np.uint16) == int(bits, 16)


def test_ties_are_not_decided_by_a_reciprocal():
    """The golden ties separate the definition from a multiply by fp32(1 / d): a plausible
    shortcut that an oracle must not take."""
    groups = json.load(open(GOLDEN))["groups"]
    differ = 0
    for grp in groups:
        x = _golden_group(grp)
        q, d = kvcache.quantize(x)
        inv = np.float32(1) / np.float32(d[0, 0]) if d[0, 0] > 0 else np.float32(0)
        shortcut = np.clip(np.rint(x[0].astype(np.float32) * inv), -127, 127)
        differ += int(np.count_nonzero(shortcut != q[0]))
    assert differ >= 2


def _rint_exact(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2):
        return fl + 1
    return fl


def test_codes_equal_exact_rational_rounding():
    """Brute force with exact rationals: d is the least fp16 at or above max|x| / 127 and
    q = rint(x / d) half to even, on random groups and on groups built around exact ties."""
    rng = np.random.default_rng(11)
    rows = []
    for _ in range(48):
        rows.append(rng.standard_normal(32) * rng.choice([1e-5, 1e-2, 1.0, 300.0, 20000.0]))
    for _ in range(48):                                  # ties: x = (k + 1/2) d for the group's own d
        amax = float(np.float16(rng.uniform(1.0, 60000.0)))
        dd = np.float16(amax / 127)
        if float(dd) < amax / 127:
            dd = np.nextafter(dd, np.float16(np.inf))
        r = np.zeros(32)
        r[0] = amax
        ks = rng.integers(-127, 127, size=31)
        r[1:] = (ks + 0.5) * float(dd)
        rows.append(np.where(np.abs(r) <= amax, r, 0.0))
    x = np.clip(np.array(rows), -65504, 65504).astype(np.float16)
    q, d = kvcache.quantize(x)
    fp16_all = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    for i in range(x.shape[0]):
        xs = [Fraction(float(v)) for v in x[i]]
        amax = max(abs(v) for v in xs)
        t = amax / 127
        d_exact = Fraction(float(fp16_all[np.searchsorted(fp16_all, float(t) * (1 - 1e-9))]))
        while d_exact < t:                               # the least fp16 >= t, in exact arithmetic
            d_exact = Fraction(float(np.nextafter(np.float16(float(d_exact)), np.float16(np.inf))))
        assert Fraction(float(d[i, 0])) == d_exact, i
        for j, v in enumerate(xs):
            want = 0 if d_exact == 0 else max(-127, min(127, _rint_exact(v / d_exact)))
            assert int(q[i, j]) == want, (i, j, float(v), float(d_exact))


def test_error_within_half_a_step_and_codes_in_range():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 256)) * rng.choice([1e-3, 1.0, 30.0], size=(64, 1))).astype(np.float16)
    x[5, 64:96] = 0                                   # an all-zero group
    x[9, 64] = 60000.0                                # near the fp16 maximum
    q, d = kvcache.quantize(x)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    xh = kvcache.dequantize(q, d)
    step = np.repeat(d.astype(np.float64), 32, axis=1)
    err = np.abs(xh.astype(np.float64) - x.astype(np.float64))
    assert np.all(err <= step / 2 * (1 + 1e-6) + 1e-30)
    assert np.all(q[5, 64:96] == 0) and d[5, 2] == 0
    # d is the smallest fp16 at or above max|x| / 127 (the grid covers every group)
    amax = np.abs(x.astype(np.float64)).reshape(64, 8, 32).max(axis=2)
    assert np.all(d.astype(np.float64) >= amax / 127 * (1 - 1e-6))
    below = np.nextafter(d, np.float16(0)).astype(np.float64)
    assert np.all((d == 0) | (below < amax / 127 * (1 + 1e-6)))


def test_fp16_decode_is_finite_and_saturates_at_the_fp16_maximum():
    x = np.zeros((3, 32), np.float16)
    x[0, :] = 65504.0
    x[0, 1::2] = -65504.0
    x[1, 0] = 65504.0
    x[1, 1:] = np.linspace(-65000, 65000, 31).astype(np.float16)
    x[2, 0] = 65440.0                                 # d = 515.5: 127 d = 65468.5, no saturation
    q, d = kvcache.quantize(x)
    assert float(d[0, 0]) == 516.0 and float(d[2, 0]) == 515.5
    xh = kvcache.dequantize_fp16(q, d)
    assert np.all(np.isfinite(xh.astype(np.float32)))
    assert np.all(xh[0, ::2] == np.float16(65504.0)) and np.all(xh[0, 1::2] == np.float16(-65504.0))
    err = np.abs(xh.astype(np.float64) - x.astype(np.float64))
    half = np.repeat(d.astype(np.float64), 32, axis=1) / 2
    assert np.all(err[0] <= half[0])                  # saturated codes: within d/2 exactly
    # elsewhere one fp16 rounding of d * q adds at most half an fp16 unit (32 / 2 up here)
    assert np.all(err <= half + 16.0)
    assert xh[2, 0] == np.float16(65472.0) and q[2, 0] == 127


def test_one_hot_groups_decode_to_full_scale():
    x = np.zeros((3, 32), np.float16)
    x[0, 3], x[1, 31], x[2, 0] = 3.0, -0.125, 100.0
    q, d = kvcache.quantize(x)
    assert q[0, 3] == 127 and q[1, 31] == -127 and q[2, 0] == 127
    assert np.count_nonzero(q) == 3
