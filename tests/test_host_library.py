"""CPU tests of libqgemv's host side: symbol exports, bitstreams, the eight quantizers against
the oracle (byte-exact canonical encodings), the device-layout permutation and error codes.

No GPU work is launched here. The oracle and the library share no code: agreement of their
canonical bytes is agreement of two independent implementations of the same spec.
"""
import ctypes

import numpy as np
import pytest

import dequant_gemv_q4g32_amd as qg
from oracle import bitstream, int4
from oracle import groupwise as gw
from oracle import superblock as sb
from workloads import laplace_weights, uniform_codes

FMTS = ["q4g32", "q2sb", "q3sb", "q5sb", "q6sb", "q4g16", "q4g64", "q4g128", "q4a32", "q4g32h",
        "q2sb_bf16", "q3sb_bf16", "q5sb_bf16", "q6sb_bf16", "q3g32", "q5g32", "q3sb_planes"]


def oracle_canonical(fmt, w):
    if fmt in gw.BITS:
        codes, s, m = gw.encode(fmt, w)
        return np.concatenate([codes.reshape(-1), s.reshape(-1).view(np.uint8), m.reshape(-1).view(np.uint8)])
    if fmt == "q4g32h":
        codes, s16 = int4.encode_h(w)
        return np.concatenate([codes.reshape(-1), s16.reshape(-1).view(np.uint8)])
    if fmt == "q4a32":
        codes, scales, zeros = int4.encode_asym(w)
        return np.concatenate([codes.reshape(-1), scales.reshape(-1).view(np.uint8), zeros.reshape(-1)])
    if fmt in qg.Q4_GROUPS:
        codes, scales = int4.encode(w, qg.Q4_GROUPS[fmt])
        return np.concatenate([codes.reshape(-1), scales.reshape(-1).view(np.uint8)])
    return sb.encode(fmt, w).reshape(-1)


def test_exports_every_declared_symbol():
    names = qg.declared_functions()
    assert len(names) >= 27
    for name in names:
        assert hasattr(qg.lib, name), name
    assert qg.lib.qg_abi_version() == 1


def test_strerror():
    assert qg.lib.qg_strerror(0) == b"ok"
    for st in range(-8, 0):
        assert qg.lib.qg_strerror(st) != b"unknown status"


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
def test_bitstreams_match_oracle(bits):
    codes = uniform_codes(4099, bits, seed=300 + bits)
    got = qg.pack_bits(bits, codes)
    want = bitstream.pack_bits(codes, bits)
    assert np.array_equal(got, want)
    assert np.array_equal(qg.unpack_bits(bits, got, codes.size), codes)
    if bits < 8:
        bad = codes.copy()
        bad[17] = 1 << bits
        with pytest.raises(qg.QGError):
            qg.pack_bits(bits, bad)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape,seed,outl", [((7, 512), 1, 0.0), ((33, 1024), 2, 0.01), ((5, 4352), 3, 0.001)])
def test_quantizer_matches_oracle(fmt, shape, seed, outl):
    w = laplace_weights(*shape, 0.02, seed, outlier_frac=outl)
    got = qg.quantize(fmt, w)
    want = oracle_canonical(fmt, w)
    assert got.shape == want.shape
    diff = np.nonzero(got != want)[0]
    assert diff.size == 0, f"{diff.size} bytes differ, first at {diff[:5]}"


@pytest.mark.parametrize("fmt", FMTS)
def test_quantizer_edge_blocks_match_oracle(fmt):
    k = 768
    w = laplace_weights(6, k, 0.02, 17, outlier_frac=0.01)
    w[0, :] = 0.0                                  # all-zero row
    w[1, 256:512] = np.float32(0.0125)             # constant super-block
    w[2, 0:32] = np.abs(w[2, 0:32])                # positive-only groups
    w[3, 32:64] = -np.abs(w[3, 32:64])             # negative-only groups
    w[4, 5] = np.float32(6e4)                      # large but representable
    w[5, ::7] = np.float32(1e-30)                  # tiny values
    assert np.array_equal(qg.quantize(fmt, w), oracle_canonical(fmt, w))


def test_q4g32_ragged_k():
    w = laplace_weights(3, 96, 0.02, 5)           # k % 64 == 32
    assert np.array_equal(qg.quantize("q4g32", w), oracle_canonical("q4g32", w))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(1, 256), (9, 1280), (4, 4352), (2, 11008)])
def test_device_layout_round_trip_and_sizes(fmt, n, k):
    w = laplace_weights(n, k, 0.02, n + k)
    can = qg.quantize(fmt, w)
    lay = qg.device_layout(fmt, n, k)
    assert lay.algorithmic_bytes == can.size == qg.canonical_bytes(fmt, n, k)
    assert lay.total_bytes - lay.algorithmic_bytes < 1024
    for p in range(lay.nplanes):
        assert lay.plane_offset[p] % 256 == 0
    dev = qg.to_device_layout(fmt, can, n, k)
    assert dev.size == lay.total_bytes
    assert np.array_equal(qg.from_device_layout(fmt, dev, n, k), can)
    # a pure bit permutation: the number of set bits is preserved
    assert np.unpackbits(dev).sum() == np.unpackbits(can).sum()


def test_device_layout_q4g32_ragged():
    w = laplace_weights(5, 160, 0.02, 8)
    can = qg.quantize("q4g32", w)
    dev = qg.to_device_layout("q4g32", can, 5, 160)
    assert np.array_equal(qg.from_device_layout("q4g32", dev, 5, 160), can)


@pytest.mark.parametrize("fmt", FMTS)
def test_algorithmic_bytes_match_oracle(fmt):
    n, k = 64, 4096
    if fmt == "q4a32":
        want = int4.algorithmic_bytes_asym(n, k)
    elif fmt == "q4g32h":
        want = int4.algorithmic_bytes_h(n, k)
    elif fmt in gw.BITS:
        want = gw.algorithmic_bytes(fmt, n, k)
    else:
        want = int4.algorithmic_bytes(n, k, qg.Q4_GROUPS[fmt]) if fmt in qg.Q4_GROUPS else sb.algorithmic_bytes(fmt, n, k)
    assert qg.device_layout(fmt, n, k).algorithmic_bytes == want


def test_error_codes():
    w = np.zeros((2, 256), np.float32)
    with pytest.raises(qg.QGError) as e:
        qg.quantize("q3sb", np.zeros((2, 200), np.float32))
    assert e.value.status == -2
    bad = w.copy()
    bad[1, 3] = np.nan
    for fmt in FMTS:
        with pytest.raises(qg.QGError) as e:
            qg.quantize(fmt, bad)
        assert e.value.status == -4
    big = w.copy()
    big[0, 0] = np.float32(1e10)
    for fmt in ("q2sb", "q3sb", "q5sb", "q6sb", "q4g32h"):
        with pytest.raises(qg.QGError) as e:
            qg.quantize(fmt, big)
        assert e.value.status == -5
    assert qg.lib.qg_quantize(19, None, 1, 256, 256, None) == -6
    for fmt in ("q2sb_bf16", "q3sb_bf16", "q5sb_bf16", "q6sb_bf16"):      # bf16 covers 1e10
        assert np.array_equal(qg.quantize(fmt, big), oracle_canonical(fmt, big))
    out = ctypes.c_int64()
    assert qg.lib.qg_canonical_bytes(3, 1, 100, ctypes.byref(out)) == -2
    assert qg.lib.qg_canonical_bytes(4, 1, 96, ctypes.byref(out)) == 0 and out.value == 48 + 12
    assert qg.lib.qg_canonical_bytes(10, 2, 128, ctypes.byref(out)) == 0 and out.value == 2 * (64 + 16 + 4)
    assert qg.lib.qg_canonical_bytes(10, 1, 96, ctypes.byref(out)) == -2


def test_packed_bytes_gives_both_sizes():
    """qg_packed_bytes: the allocation size of the device layout and the algorithmic bytes (the
    canonical size: the byte table's 110 B per 256 weights for q3sb, 20 B per 32 INT4 weights)."""
    tot, alg = ctypes.c_int64(), ctypes.c_int64()
    assert qg.lib.qg_packed_bytes(3, 4096, 4096, ctypes.byref(tot), ctypes.byref(alg)) == 0
    assert alg.value == 4096 * 16 * 110
    lay = qg.device_layout("q3sb", 4096, 4096)
    assert tot.value == lay.total_bytes and alg.value == lay.algorithmic_bytes
    assert qg.lib.qg_packed_bytes(4, 4096, 4096, None, ctypes.byref(alg)) == 0 and alg.value == 4096 * 128 * 20
    assert qg.lib.qg_packed_bytes(4, 4096, 4096, ctypes.byref(tot), None) == 0
    assert qg.lib.qg_packed_bytes(3, 1, 100, ctypes.byref(tot), ctypes.byref(alg)) == -2
    assert qg.lib.qg_packed_bytes(19, 1, 256, ctypes.byref(tot), ctypes.byref(alg)) == -6


def test_device_entry_points_validate_without_launching():
    """Argument errors are returned before any HIP call, so they are checkable without a GPU."""
    L = qg.lib
    assert L.qg_gemv(3, None, None, None, 0, 4, 100, None) == -2          # k % 256
    assert L.qg_gemv(4, None, None, None, 0, 4, 48, None) == -2           # k % 32
    assert L.qg_gemv(10, None, None, None, 0, 4, 96, None) == -2          # q4a32: k % 64
    assert L.qg_gemv(19, None, None, None, 0, 4, 256, None) == -6          # format
    assert L.qg_gemv(3, None, None, None, 0, 0, 256, None) == 0           # n == 0: no-op
    assert L.qg_gemv(3, None, None, None, 0, 4, 256, None) == -1          # null
    assert L.qg_gemv(3, 256, 16, 3, 0, 4, 256, None) == -3                # y misaligned
    assert L.qg_gemv(3, 257, 16, 2, 0, 4, 256, None) == -3                # w misaligned
    assert L.qg_gemv(3, 256, 18, 2, 0, 4, 256, None) == -3                # x misaligned
    assert L.qg_gemv(3, 256, 16, 2, 0, 4, (1 << 20) + 256, None) == -2    # k too long
    assert L.qg_gemv(4, 256, 16, 2, 0, (1 << 23) + 1, 1024, None) == -2   # 4 GiB code plane
    assert L.qg_dequantize(3, None, None, None, 4, 256, None) == -1
    assert L.qg_dequantize(5, 256, None, 16, 4, 100, None) == -2
    assert L.qg_gemv_batched(2, 256, 100, 16, 0, 2, 4, 0, 3, 4, 256, None) == -3   # w stride
    # qg_gemm(fmt, w, X, ldx, Y, ldy, y_f32, m, n, k, stream)
    assert L.qg_gemm(3, 256, 16, 256, 2, 4, 0, 0, 4, 256, None) == 0      # m == 0: no-op
    assert L.qg_gemm(3, 256, 16, 256, 2, 4, 0, -1, 4, 256, None) == -2    # m < 0
    assert L.qg_gemm(3, 256, 16, 128, 2, 4, 0, 2, 4, 256, None) == -2     # ldx < k
    assert L.qg_gemm(3, 256, 16, 256, 2, 3, 0, 2, 4, 256, None) == -2     # ldy < n
    assert L.qg_gemm(3, 256, 16, 260, 2, 4, 0, 2, 4, 256, None) == -3     # ldx % 8
    assert L.qg_gemm(3, 256, 16, 1 << 22, 2, 4, 0, 20, 4, 256, None) == -2    # prefill: ldx >= 2^22
    assert L.qg_gemm(3, 256, 16, 1 << 26, 2, 4, 0, 8, 4, 256, None) == -2     # 5..16 rows: ldx >= 2^26
    assert L.qg_gemm(3, None, 16, 256, 2, 4, 0, 2, 4, 256, None) == -1    # null w
    assert L.qg_gemm(5, 256, 16, 256, 2, 4, 0, 2, 4, 100, None) == -2     # k % 256
    assert L.qg_gemm(19, 256, 16, 256, 2, 4, 0, 2, 4, 256, None) == -6     # format
    assert L.dequant_gemm_q6sb(256, 16, 256, 3, 4, 2, 4, 256, None) == -3  # Y misaligned


def test_grouped_entry_point_validates_every_matrix_first():
    """qg_gemm_grouped checks all matrices before launching anything: an error in the last
    matrix is returned even though the first ones are valid (no GPU needed)."""
    import ctypes
    L = qg.lib
    vp, i64 = ctypes.c_void_p, ctypes.c_int64

    def call(fmt, ws, xs, ys, ns, ks, m=1, ldx=None, ldy=None, count=None):
        c = len(ws) if count is None else count
        arr = lambda t, v: (t * max(len(v), 1))(*v)
        return L.qg_gemm_grouped(fmt, c, arr(vp, ws), arr(vp, xs), arr(i64, ldx or ks), arr(vp, ys),
                                 arr(i64, ldy or ns), arr(i64, ns), arr(i64, ks), m, 0, None)

    ok = dict(ws=[256, 512], xs=[16, 32], ys=[2, 4], ns=[4, 8], ks=[256, 512])
    assert call(3, **{**ok, "ks": [256, 100]}) == -2                      # k % 256 in matrix 1
    assert call(4, **{**ok, "ks": [256, 48]}) == -2                       # k % 32
    assert call(3, **{**ok, "ws": [256, 300]}) == -3                      # w misaligned
    assert call(3, **{**ok, "xs": [16, 18]}) == -3                        # x misaligned
    assert call(3, **{**ok, "ys": [2, 3]}) == -3                          # y misaligned
    assert call(3, **{**ok, "ws": [256, 0]}) == -1                        # null w
    assert call(3, **{**ok, "ks": [256, (1 << 20) + 256]}) == -2          # k too long
    assert call(3, **ok, m=9) == -2                                       # m > 8
    assert call(3, **ok, m=-1) == -2
    assert call(3, **ok, m=2, ldx=[256, 500]) == -2                       # ldx < k
    assert call(3, **ok, m=2, ldy=[4, 7]) == -2                           # ldy < n
    assert call(3, **ok, m=2, ldx=[260, 512]) == -3                       # ldx % 8
    assert call(19, **ok) == -6                                            # format
    assert call(3, [256] * 9, [16] * 9, [2] * 9, [4] * 9, [256] * 9) == -2   # more than 8
    assert call(3, **ok, m=0) == 0                                        # m == 0: no-op
    assert call(3, **{**ok, "ns": [0, 0]}) == 0                           # n == 0: no-op
    assert L.qg_gemm_grouped(3, 0, None, None, None, None, None, None, None, 1, 0, None) == 0
    assert L.qg_gemm_grouped(3, 1, None, None, None, None, None, None, None, 1, 0, None) == -1


def test_act_order_entry_point_validates_without_launching():
    L = qg.lib
    # qg_gemm_act_order(fmt, w, X, ldx, perm, Y, ldy, y_f32, m, n, k, stream)
    assert L.qg_gemm_act_order(3, 256, 16, 256, None, 2, 4, 0, 1, 4, 256, None) == -1    # null perm
    assert L.qg_gemm_act_order(3, 256, 16, 256, 52, 2, 4, 0, 1, 4, 256, None) == -3      # perm misaligned
    assert L.qg_gemm_act_order(3, 256, 16, 256, 32, 2, 4, 0, 9, 4, 256, None) == -2      # m > 8
    assert L.qg_gemm_act_order(3, 256, 16, 256, 32, 2, 4, 0, 1, 4, 100, None) == -2      # k % 256
    assert L.qg_gemm_act_order(3, 256, 16, 128, 32, 2, 4, 0, 2, 4, 256, None) == -2      # ldx < k
    assert L.qg_gemm_act_order(19, 256, 16, 256, 32, 2, 4, 0, 1, 4, 256, None) == -6      # format
    assert L.qg_gemm_act_order(3, 256, 16, 256, 32, 2, 4, 0, 0, 4, 256, None) == 0       # m == 0


def test_kv_codec_entry_points_validate_without_launching():
    L = qg.lib
    # qg_kv_quantize(src, ld_src, rows, cols, codes, scales, stream)
    assert L.qg_kv_quantize(16, 64, 2, 48, 8, 2, None) == -2          # cols % 32
    assert L.qg_kv_quantize(16, 16, 2, 32, 8, 2, None) == -2          # ld_src < cols
    assert L.qg_kv_quantize(18, 64, 2, 64, 8, 2, None) == -3          # src misaligned
    assert L.qg_kv_quantize(16, 68, 2, 64, 8, 2, None) == -3          # ld_src % 8
    assert L.qg_kv_quantize(16, 64, 2, 64, 12, 2, None) == -3         # codes misaligned
    assert L.qg_kv_quantize(None, 64, 2, 64, 8, 2, None) == -1
    assert L.qg_kv_quantize(16, 64, 0, 64, 8, 2, None) == 0           # no rows: no-op
    # qg_kv_dequantize(codes, scales, rows, cols, dst, ld_dst, stream)
    assert L.qg_kv_dequantize(8, 2, 2, 40, 16, 64, None) == -2
    assert L.qg_kv_dequantize(8, 3, 2, 64, 16, 64, None) == -3        # scales misaligned
    assert L.qg_kv_dequantize(8, 2, 2, 64, None, 64, None) == -1
    assert L.qg_kv_dequantize(8, 2, -1, 64, 16, 64, None) == -2
