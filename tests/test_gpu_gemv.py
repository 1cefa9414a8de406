"""GPU parity tests for the dequant GEMV and the device decode, against the oracle.

Bar: decoded codes bit-exact; decoded fp32 weights exactly float32(W_hat) (single-rounding
products); GEMV outputs within 2e-3 * sum_k |W_hat[r,k] x[k]| per row (fp16 and fp32 output).
Inputs are seeded Laplace weights and fp16 normal activations from workloads.py.
"""
import numpy as np
import pytest

import dequant_gemv_q4g32_amd as qg
from gpu_util import assert_close, device_weights, oracle_decode, oracle_y
from workloads import WORKLOADS, activations, laplace_weights

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FMTS = ["q4g32", "q2sb", "q3sb", "q5sb", "q6sb", "q4g16", "q4g64", "q4g128", "q4a32", "q4g32h",
        "q2sb_bf16", "q3sb_bf16", "q5sb_bf16", "q6sb_bf16", "q3g32", "q5g32", "q3sb_planes"]
# (n, k): several tiles, ragged n, K split over 1, 2, 3 and 7 waves
SHAPES = [(37, 512), (16, 256), (1001, 1024), (64, 4096), (20, 4352), (9, 8192), (33, 11008), (5, 28672)]


def _x(k, seed, m=1):
    return activations(m, k, seed)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(37, 512), (5, 4352), (3, 11008)])
def test_dequantize_bit_exact(fmt, n, k):
    w = laplace_weights(n, k, 0.02, n * 7 + k, outlier_frac=0.002)
    codes_ref, w_hat = oracle_decode(fmt, w)
    wd = device_weights(fmt, w)
    vals, codes = qg.dequantize(fmt, wd, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), codes_ref)
    assert np.array_equal(vals.cpu().numpy(), w_hat.astype(np.float32))


@pytest.mark.parametrize("n,k", [(7, 96), (4, 4128), (3, 160)])
def test_dequantize_q4g32_ragged_k(n, k):
    w = laplace_weights(n, k, 0.02, k)
    codes_ref, w_hat = oracle_decode("q4g32", w)
    vals, codes = qg.dequantize("q4g32", device_weights("q4g32", w), n, k)
    assert np.array_equal(codes.cpu().numpy(), codes_ref)
    assert np.array_equal(vals.cpu().numpy(), w_hat.astype(np.float32))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", SHAPES)
def test_gemv_matches_oracle(fmt, n, k):
    w = laplace_weights(n, k, 0.02, 31 * n + k, outlier_frac=0.001)
    _, w_hat = oracle_decode(fmt, w)
    x = _x(k, n + 3 * k)
    y_ref, bound = oracle_y(w_hat, x)
    wd = device_weights(fmt, w)
    xd = torch.from_numpy(x[0]).cuda()
    y16 = qg.gemv(fmt, wd, xd, n, k)
    y32 = qg.gemv(fmt, wd, xd, n, k, out_f32=True)
    torch.cuda.synchronize()
    assert_close(y32.cpu().numpy()[None, :], y_ref, bound, f"{fmt} {n}x{k} f32")
    assert_close(y16.cpu().float().numpy()[None, :], y_ref, bound, f"{fmt} {n}x{k} f16")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(7, 96), (9, 4128)])
def test_gemv_q4g32_ragged_or_sb(fmt, n, k):
    if fmt != "q4g32":
        k = 256 * max(1, k // 256)
    w = laplace_weights(n, k, 0.02, k + 1)
    _, w_hat = oracle_decode(fmt, w)
    x = _x(k, k + 2)
    y_ref, bound = oracle_y(w_hat, x)
    y = qg.gemv(fmt, device_weights(fmt, w), torch.from_numpy(x[0]).cuda(), n, k, out_f32=True)
    assert_close(y.cpu().numpy()[None, :], y_ref, bound, f"{fmt} {n}x{k}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_one_hot_columns(fmt):
    """x = e_c selects column c of W_hat: pins the position of every decoded column."""
    n, k = 24, 512 if fmt != "q4g32" else 480
    w = laplace_weights(n, k, 0.02, 99)
    _, w_hat = oracle_decode(fmt, w)
    wd = device_weights(fmt, w)
    xs = np.zeros((k, k), np.float16)
    np.fill_diagonal(xs, 1.0)
    xd = torch.from_numpy(xs).cuda()
    y = torch.empty((k, n), dtype=torch.float32, device="cuda")
    qg.gemv_batched(fmt, wd, 0, xd, y, k, n, k)
    got = y.cpu().numpy()                      # [c, r] = W_hat[r, c]
    want = w_hat.T
    assert np.all(np.abs(got - want) <= 2e-3 * np.abs(want)), np.argwhere(np.abs(got - want) > 2e-3 * np.abs(want))[:5]


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_zero_x_and_empty(fmt):
    n, k = 10, 1024
    wd = device_weights(fmt, laplace_weights(n, k, 0.02, 5))
    y = qg.gemv(fmt, wd, torch.zeros(k, dtype=torch.float16, device="cuda"), n, k, out_f32=True)
    assert torch.all(y == 0).item()
    y0 = torch.full((n,), 7.0, dtype=torch.float16, device="cuda")
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    qg.gemv(fmt, dummy, torch.zeros(8, dtype=torch.float16, device="cuda"), n, 0, out=y0)
    assert torch.all(y0 == 0).item()


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_batched_equals_single(fmt):
    n, k, cnt = 300, 2048, 5
    lay = qg.device_layout(fmt, n, k)
    stride = (lay.total_bytes + 255) // 256 * 256
    buf = torch.zeros(stride * cnt, dtype=torch.uint8, device="cuda")
    xs = _x(k, 4, m=cnt)
    ref = []
    for b in range(cnt):
        w = laplace_weights(n, k, 0.02, 1000 + b)
        wd = device_weights(fmt, w)
        buf[b * stride:b * stride + lay.total_bytes].copy_(wd)
        ref.append(qg.gemv(fmt, wd, torch.from_numpy(xs[b]).cuda(), n, k, out_f32=True))
    y = torch.empty((cnt, n), dtype=torch.float32, device="cuda")
    qg.gemv_batched(fmt, buf, stride, torch.from_numpy(xs).cuda(), y, cnt, n, k)
    for b in range(cnt):
        assert torch.equal(y[b], ref[b])


def _sampled_rows(n, seed, count=48):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(n, count), replace=False)]))
    return rows


def _full_cases():
    cases = []
    for name, wl in WORKLOADS.items():
        if wl.m != 1:
            continue
        seen = set()
        for i, shape in enumerate(wl.shapes):
            if shape not in seen:            # each distinct shape once
                seen.add(shape)
                cases.append((name, i))
    return cases


FULL = _full_cases()


@pytest.mark.parametrize("name,i", FULL, ids=[f"{n}-{i}" for n, i in FULL])
def test_full_size_workloads_sampled_rows(name, i):
    """The full-size matrices in the launch configuration the benchmark times; the oracle
    recomputes a sample of rows one by one (rows are independent)."""
    wl = WORKLOADS[name]
    n, k = wl.shapes[i]
    w = wl.weights(i)
    x = wl.x(i)
    wd = device_weights(wl.fmt, w)
    y = qg.gemv(wl.fmt, wd, torch.from_numpy(x[0]).cuda(), n, k)
    rows = _sampled_rows(n, i)
    _, w_hat = oracle_decode(wl.fmt, w[rows])
    y_ref, bound = oracle_y(w_hat, x)
    torch.cuda.synchronize()
    assert_close(y.cpu().float().numpy()[rows][None, :], y_ref, bound, f"{name}[{i}]")


def test_q4a32_zero_points_over_their_range():
    """Asymmetric INT4: groups shifted from all-negative to all-positive, so that the zero
    points take every value 0..15; decode bit-exact, GEMV (1 and 4 rows) and prefill (64 rows)
    within the tolerance."""
    n, k = 48, 2048
    w = laplace_weights(n, k, 0.01, 404)
    shift = np.linspace(-0.06, 0.06, n * (k // 32), dtype=np.float32).reshape(n, k // 32)
    w = (w + np.repeat(shift, 32, axis=1)).astype(np.float32)
    codes_ref, w_hat = oracle_decode("q4a32", w)
    from oracle import int4
    zeros = int4.quantize_asym(w)[2]
    assert set(np.unique(zeros)) == set(range(16))
    wd = device_weights("q4a32", w)
    vals, codes = qg.dequantize("q4a32", wd, n, k)
    assert np.array_equal(codes.cpu().numpy(), codes_ref)
    assert np.array_equal(vals.cpu().numpy(), w_hat.astype(np.float32))
    for m in (1, 4, 64):
        x = _x(k, 405 + m, m)
        y_ref, bound = oracle_y(w_hat, x)
        y = qg.gemm("q4a32", wd, torch.from_numpy(x).cuda(), n, k, out_f32=True)
        assert_close(y.cpu().numpy(), y_ref, bound, f"q4a32 m={m}")


@pytest.mark.parametrize("fmt", ["q2sb_bf16", "q3sb_bf16", "q5sb_bf16", "q6sb_bf16"])
def test_bf16_super_scales_past_the_fp16_range(fmt):
    """bf16 super-scales: rows with super-blocks whose scale would overflow fp16 (weights of
    order 1e8) beside ordinary ones; decode bit-exact, outputs (fp32) within the tolerance
    for 1, 2 and 4 activation rows through qg_gemm and 8 through the grouped entry point (the
    streaming kernel: the matrix-core paths take W_hat through fp16, whose range such weights
    exceed)."""
    n, k = 40, 1024
    w = laplace_weights(n, k, 0.02, 77)
    w[3, 300] = np.float32(2.0e8)
    w[17, 5:40] *= np.float32(3.0e9)
    codes_ref, w_hat = oracle_decode(fmt, w)
    wd = device_weights(fmt, w)
    vals, codes = qg.dequantize(fmt, wd, n, k)
    assert np.array_equal(codes.cpu().numpy(), codes_ref)
    assert np.array_equal(vals.cpu().numpy(), w_hat.astype(np.float32))
    for m in (1, 2, 4, 8):
        x = _x(k, 78 + m, m)
        y_ref, bound = oracle_y(w_hat, x)
        if m <= 4:
            y = qg.gemm(fmt, wd, torch.from_numpy(x).cuda(), n, k, out_f32=True)
        else:
            y = torch.empty((m, n), dtype=torch.float32, device="cuda")
            qg.gemm_grouped(fmt, [wd], [torch.from_numpy(x).cuda()], [(n, k)], outs=[y])
        assert_close(y.cpu().numpy(), y_ref, bound, f"{fmt} m={m}")


def test_headline_launch_configuration_sampled_rows():
    """The benchmark's exact launch: 32 independent q3sb 4096 x 4096 GEMVs in one strided
    batch (each with its own activations); sampled rows of several members against the
    oracle."""
    wl = WORKLOADS["q3sb_gemv_4096"]
    n, k = wl.shapes[0]
    w = wl.weights(0)
    wd = device_weights(wl.fmt, w)
    lay = qg.device_layout(wl.fmt, n, k)
    stride = (lay.total_bytes + 255) // 256 * 256
    count = 32
    buf = torch.zeros(count * stride, dtype=torch.uint8, device="cuda")
    for c in range(count):
        buf[c * stride:c * stride + lay.total_bytes].copy_(wd)
    xs = activations(count, k, 4242)
    ys = torch.empty((count, n), dtype=torch.float16, device="cuda")
    qg.gemv_batched(wl.fmt, buf, stride, torch.from_numpy(xs).cuda(), ys, count, n, k)
    rows = _sampled_rows(n, 0)
    _, w_hat = oracle_decode(wl.fmt, w[rows])
    torch.cuda.synchronize()
    y = ys.cpu().float().numpy()
    for b in (0, 17, 31):
        y_ref, bound = oracle_y(w_hat, xs[b:b + 1])
        assert_close(y[b, rows][None, :], y_ref, bound, f"member {b}")


def test_read_probe_streams_without_writing():
    """The read-ceiling probe reads any multiple of 16 bytes (one-shot and grid-stride sizes,
    a ragged tail of 16-byte chunks) and leaves the sink alone (zeros xor to 0); bad sizes
    are rejected."""
    buf = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    for nbytes in (16, 16 * 1023, 16 * 1025, 48 << 20, (64 << 20) - 16 * 37):
        qg.read_probe(buf, nbytes, sink)
    torch.cuda.synchronize()
    assert sink.item() == 7
    for bad in (8, -16):
        with pytest.raises(Exception):
            qg.read_probe(buf, bad, sink)
