"""Pins for oracle/kvcache.py (8-bit KV-cache groups: "二三五六位量化" page, section 4.1)."""
import json
import os

import numpy as np

from oracle import kvcache

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kvcache_groups.json")


def test_page_byte_arithmetic():
    g = json.load(open(GOLDEN))["sizes"]
    n = kvcache.kv_cache_elements(32, 8, 128, 8192)
    assert n == g["elements"]
    assert n * 2 == g["fp16_bytes"]                   # the page's 1.07 GB
    assert n * kvcache.bytes_per_element() == g["int8_bytes"]
    assert abs(kvcache.bytes_per_element() - 1.06) < 0.005   # the page's "about 1.06"


def test_hand_worked_groups():
    for grp in json.load(open(GOLDEN))["groups"]:
        x = np.zeros((1, 32), np.float16)
        for i, v in grp["values"].items():
            x[0, int(i)] = v
        q, d = kvcache.quantize(x)
        assert d[0, 0].view(np.uint16) == int(grp["scale_bits"], 16), (grp, hex(d[0, 0].view(np.uint16)))
        want = np.zeros(32, np.int8)
        for i, c in grp["codes"].items():
            want[int(i)] = c
        assert np.array_equal(q[0], want), (q[0], want)


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


def test_one_hot_groups_decode_to_full_scale():
    x = np.zeros((3, 32), np.float16)
    x[0, 3], x[1, 31], x[2, 0] = 3.0, -0.125, 100.0
    q, d = kvcache.quantize(x)
    assert q[0, 3] == 127 and q[1, 31] == -127 and q[2, 0] == 127
    assert np.count_nonzero(q) == 3
