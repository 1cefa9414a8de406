"""GPU parity tests for the 8-bit KV-cache group codec (qg_kv_quantize / qg_kv_dequantize)
against the oracle ("二三五六位量化" page section 4.1; readings in oracle/kvcache.py).

Bar: bit-exact. The codes and fp16 scales are integer decisions with one correct answer (the
oracle takes them on exact quotients), and the decoded value d * q is exact before its one
saturating rounding to fp16, so every code, scale and decoded fp16 must equal the oracle's.
Covers one group, ragged row counts, strided fp16 rows, all-zero groups, exact ties of x / d
(the golden groups), values at the fp16 maximum (finite decode within d/2) and subnormal ones,
and one full layer of the 7B-like cache (8192 tokens x 8 KV heads x 128).
"""
import json
import os

import numpy as np
import pytest

import dequant_gemv_q4g32_amd as qg
from oracle import kvcache

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _data(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * rng.choice([1e-4, 0.05, 1.0, 40.0], size=(rows, 1))
    flat = x.reshape(-1)
    flat[rng.choice(flat.size, max(1, flat.size // 500), replace=False)] *= 50.0      # outliers
    return np.clip(x, -65000, 65000).astype(np.float16)


def _roundtrip(x, ld=None):
    rows, cols = x.shape
    ld = ld or cols
    xb = torch.zeros((rows, ld), dtype=torch.float16, device="cuda")
    xb[:, :cols] = torch.from_numpy(x).cuda()
    codes, scales = qg.kv_quantize(xb[:, :cols])
    outb = torch.full((rows, ld), 9.0, dtype=torch.float16, device="cuda")
    qg.kv_dequantize(codes, scales, out=outb[:, :cols])
    torch.cuda.synchronize()
    ob = outb.cpu().numpy()
    assert np.all(ob[:, cols:] == 9.0), "dequantize wrote outside dst[:, :cols]"
    return codes.cpu().numpy(), scales.cpu().numpy(), ob[:, :cols]


@pytest.mark.parametrize("rows,cols,ld", [(1, 32, None), (7, 96, None), (513, 1024, 1048), (64, 4096, None)])
def test_kv_codec_bit_exact_against_oracle(rows, cols, ld):
    x = _data(rows, cols, rows * 7 + cols)
    q, d, xh = _roundtrip(x, ld)
    q_ref, d_ref = kvcache.quantize(x)
    assert np.array_equal(d.view(np.uint16), d_ref.view(np.uint16)), "scales differ"
    assert np.array_equal(q, q_ref), f"codes differ at {np.argwhere(q != q_ref)[:5]}"
    xh_ref = kvcache.dequantize_fp16(q_ref, d_ref)
    assert np.array_equal(xh.view(np.uint16), xh_ref.view(np.uint16)), "decoded values differ"


def test_kv_codec_special_groups():
    x = np.zeros((4, 128), np.float16)
    x[0, :32] = 65504.0                      # fp16 maximum
    x[0, 33] = -65504.0
    x[1, 32:64] = np.float16(6e-8)           # subnormal inputs: d rounds up to the smallest subnormal
    x[1, 64] = np.float16(-3e-5)
    x[2, 100] = 1.0                          # one-hot group
    # row 3 and most groups stay zero: d = 0, q = 0, decoded 0
    q, d, xh = _roundtrip(x)
    q_ref, d_ref = kvcache.quantize(x)
    assert np.array_equal(d.view(np.uint16), d_ref.view(np.uint16))
    assert np.array_equal(q, q_ref)
    assert np.array_equal(xh.view(np.uint16), kvcache.dequantize_fp16(q_ref, d_ref).view(np.uint16))
    assert np.all(q[3] == 0) and np.all(d[3] == 0) and np.all(xh[3] == 0)
    # the fp16-maximum group decodes finite, within d/2 of its inputs
    assert np.all(np.isfinite(xh.astype(np.float32)))
    err = np.abs(xh[0, :32].astype(np.float64) - x[0, :32].astype(np.float64))
    assert float(d[0, 0]) == 516.0 and np.all(err <= 516.0 / 2)
    assert xh[0, 0] == np.float16(65504.0) and xh[0, 33] == np.float16(-65504.0)


def test_kv_codec_golden_groups_and_ties():
    """Hand-worked groups, among them exact ties x = (k + 1/2) d that go to the even code."""
    golden = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kvcache_groups.json")))["groups"]
    x = np.zeros((len(golden), 32), np.float16)
    for gi, grp in enumerate(golden):
        for i, v in grp["values"].items():
            x[gi, int(i)] = v
    q, d, xh = _roundtrip(x)
    for gi, grp in enumerate(golden):
        assert d[gi, 0].view(np.uint16) == int(grp["scale_bits"], 16), grp
        want = np.zeros(32, np.int8)
        for i, c in grp["codes"].items():
            want[int(i)] = c
        assert np.array_equal(q[gi], want), (gi, q[gi], want)
        for i, bits in grp.get("fp16_decode_bits", {}).items():
            assert xh[gi, int(i)].view(np.uint16) == int(bits, 16)
    assert np.all(np.isfinite(xh.astype(np.float32)))


def test_kv_codec_full_layer_of_7b_cache():
    """K of one layer of the 7B-like cache: 8192 tokens x (8 KV heads x 128)."""
    x = _data(8192, 1024, 8192)
    q, d, xh = _roundtrip(x)
    q_ref, d_ref = kvcache.quantize(x)
    assert np.array_equal(d.view(np.uint16), d_ref.view(np.uint16))
    assert np.array_equal(q, q_ref)
    err = np.abs(kvcache.dequantize(q, d).astype(np.float64) - x.astype(np.float64))
    assert np.all(err <= np.repeat(d.astype(np.float64), 32, axis=1) / 2 * (1 + 1e-6) + 1e-30)
