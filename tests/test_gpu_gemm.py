"""GPU parity tests for the dequant GEMM with a few activation rows, against the oracle.

Bar: every output Y[i, r] within 2e-3 * sum_k |X[i,k] W_hat[r,k]| (fp16 and fp32 output).
Covers the three kernels qg_gemm routes to (the streaming kernel for 1-4 rows, built for 1,
2 and 4 rows per launch with the unused rows masked; the matrix-core decode kernel for 5-16,
and for 17-32 as two 16-row blocks per decoded fragment where estimated faster; the prefill
kernel beyond), strided X and Y, K split over several waves and over several
passes (the streaming kernel's passes at 8 rows through the grouped entry point), ragged n,
and the full-size decode workloads with 2, 4 and 8 activation rows on sampled output rows.
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
MS = [1, 2, 3, 4, 5, 8, 11, 17, 32]
# (n, k): several row blocks and a ragged tail, K over 1..8 waves, and (5, 28672) over two
# passes
SHAPES = [(37, 512), (1001, 1024), (20, 4352), (9, 8192), (5, 28672)]


def _run(fmt, wd, x, n, k, out_f32, ldx=None, ldy=None):
    m = x.shape[0]
    ldx = ldx or k
    ldy = ldy or n
    xbuf = torch.zeros((m, ldx), dtype=torch.float16, device="cuda")
    xbuf[:, :k] = torch.from_numpy(x).cuda()
    ybuf = torch.full((m, ldy), 3.0, dtype=torch.float32 if out_f32 else torch.float16, device="cuda")
    qg.gemm(fmt, wd, xbuf[:, :k], n, k, out=ybuf[:, :n])
    torch.cuda.synchronize()
    yb = ybuf.cpu().float().numpy()
    assert np.all(yb[:, n:] == 3.0), "GEMM wrote outside Y[:, :n]"
    return yb[:, :n]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", SHAPES)
def test_gemm_matches_oracle(fmt, n, k):
    w = laplace_weights(n, k, 0.02, 17 * n + k, outlier_frac=0.001)
    _, w_hat = oracle_decode(fmt, w)
    wd = device_weights(fmt, w)
    for m in MS:
        x = activations(m, k, 5 * m + k)
        y_ref, bound = oracle_y(w_hat, x)
        y32 = _run(fmt, wd, x, n, k, True)
        assert_close(y32, y_ref, bound, f"{fmt} m={m} {n}x{k} f32")
        if m in (2, 8):
            y16 = _run(fmt, wd, x, n, k, False)
            assert_close(y16, y_ref, bound, f"{fmt} m={m} {n}x{k} f16")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_strided_x_and_y(fmt):
    n, k = 70, 2048
    w = laplace_weights(n, k, 0.02, 123)
    _, w_hat = oracle_decode(fmt, w)
    wd = device_weights(fmt, w)
    for m in (2, 6):
        x = activations(m, k, 44 + m)
        y_ref, bound = oracle_y(w_hat, x)
        y = _run(fmt, wd, x, n, k, True, ldx=k + 24, ldy=n + 5)
        assert_close(y, y_ref, bound, f"{fmt} m={m} strided")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_gemm_many_k_passes(fmt, m):
    """K = 73728: 1152 units, more waves along K than one workgroup holds for every row count,
    so partial sums are carried across passes in LDS."""
    n, k = 3, 73728
    w = laplace_weights(n, k, 0.02, 555 + m)
    _, w_hat = oracle_decode(fmt, w)
    x = activations(m, k, 77 + m)
    y_ref, bound = oracle_y(w_hat, x)
    wd = device_weights(fmt, w)
    y = _run(fmt, wd, x, n, k, True)
    assert_close(y, y_ref, bound, f"{fmt} m={m} {n}x{k}")
    if m > 4:
        # qg_gemm takes the matrix-core kernel from 5 rows; the streaming kernel's passes
        # over K at 8 rows are reached through the grouped entry point
        yg = torch.empty((m, n), dtype=torch.float32, device="cuda")
        qg.gemm_grouped(fmt, [wd], [torch.from_numpy(x).cuda()], [(n, k)], outs=[yg])
        torch.cuda.synchronize()
        assert_close(yg.cpu().numpy(), y_ref, bound, f"{fmt} m={m} {n}x{k} streaming")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_q4g32_ragged_k(fmt):
    """q4g32 with K an odd multiple of 32 (a half unit at the end), for every row count."""
    if fmt != "q4g32":
        pytest.skip("ragged K is a q4g32 case")
    for n, k in ((7, 96), (9, 4128), (4, 160)):
        w = laplace_weights(n, k, 0.02, k + 9)
        _, w_hat = oracle_decode(fmt, w)
        wd = device_weights(fmt, w)
        for m in (1, 2, 3, 8):
            x = activations(m, k, k + m)
            y_ref, bound = oracle_y(w_hat, x)
            assert_close(_run(fmt, wd, x, n, k, True), y_ref, bound, f"q4g32 m={m} {n}x{k}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_rows_are_independent(fmt):
    """Row i of X = e_c for distinct columns c: each output row is one column of W_hat, so a
    mixed-up activation row or output row shows as a wrong column."""
    n, k = 24, 512
    w = laplace_weights(n, k, 0.02, 321)
    _, w_hat = oracle_decode(fmt, w)
    wd = device_weights(fmt, w)
    cols = np.array([5, 130, 257, 511, 0, 64, 300, 449])
    x = np.zeros((8, k), np.float16)
    x[np.arange(8), cols] = 1.0
    y = _run(fmt, wd, x, n, k, True)
    want = w_hat[:, cols].T
    assert np.all(np.abs(y - want) <= 2e-3 * np.abs(want))


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_zero_and_empty(fmt):
    n, k = 10, 1024
    wd = device_weights(fmt, laplace_weights(n, k, 0.02, 5))
    y = _run(fmt, wd, np.zeros((4, k), np.float16), n, k, True)
    assert np.all(y == 0)
    ybuf = torch.full((3, n), 7.0, dtype=torch.float16, device="cuda")
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    qg.gemm(fmt, dummy, torch.zeros((3, 8), dtype=torch.float16, device="cuda"), n, 0, out=ybuf)
    assert torch.all(ybuf == 0).item()
    ybuf.fill_(7.0)
    qg.gemm(fmt, wd, torch.zeros((0, k), dtype=torch.float16, device="cuda"), n, k, out=ybuf[:0])
    assert torch.all(ybuf == 7.0).item()


def _sampled_rows(n, seed, count=32):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(n, count), replace=False)]))


def _full_cases():
    """(format, shape index, [workload names]) for the decode-batch workloads, grouped so that
    the workloads that share a weight matrix (same format, shapes and seed) upload it once."""
    groups = {}
    for name, wl in WORKLOADS.items():
        if wl.m < 2 or wl.m > 8:
            continue
        for i in range(len(wl.shapes)):
            groups.setdefault((wl.fmt, wl.shapes, wl.seed, i), []).append(name)
    return [(key[0], key[3], names) for key, names in groups.items()]


FULL = _full_cases()


@pytest.mark.parametrize("fmt,i,names", FULL, ids=[f"{f}-{i}" for f, i, _ in FULL])
def test_full_size_small_m_sampled_rows(fmt, i, names):
    """Full-size decode-batch matrices with 2, 4 and 8 activation rows, in the launch
    configuration the library uses for them; the oracle recomputes sampled output rows."""
    wl0 = WORKLOADS[names[0]]
    n, k = wl0.shapes[i]
    w = wl0.weights(i)
    wd = device_weights(fmt, w)
    rows = _sampled_rows(n, i)
    _, w_hat = oracle_decode(fmt, w[rows])
    del w
    for name in names:
        x = WORKLOADS[name].x(i)
        y = qg.gemm(fmt, wd, torch.from_numpy(x).cuda(), n, k)
        y_ref, bound = oracle_y(w_hat, x)
        torch.cuda.synchronize()
        assert_close(y.cpu().float().numpy()[:, rows], y_ref, bound, f"{name}[{i}]")


@pytest.mark.parametrize("fmt", ["q4g32", "q3sb", "q6sb"])
def test_row_results_do_not_depend_on_launch_shape(fmt):
    """A row's output is the same fp32 sum, bit for bit, whether its wave carries one row or
    two rows per batch (large launches) and however many matrices share the launch: the
    wave reduction adds the lanes in one fixed order. The first 64 rows of an 8192-row matrix
    are quantized exactly like a 64-row matrix of the same weights (quantization is row-local)."""
    n, k = 8192, 4096
    w = laplace_weights(n, k, 0.02, 2024)
    big, small = device_weights(fmt, w), device_weights(fmt, w[:64])
    for m in (1, 2):
        x = torch.from_numpy(activations(m, k, 31 + m)).cuda()
        y_big = qg.gemm(fmt, big, x, n, k, out_f32=True)           # two rows per batch
        y_small = qg.gemm(fmt, small, x, 64, k, out_f32=True)      # one row per batch
        torch.cuda.synchronize()
        assert torch.equal(y_big[:, :64], y_small), f"{fmt} m={m}"
    # batch-1 strided batch of 8 copies (two rows per batch) against one launch per copy
    lay = qg.device_layout(fmt, n, k)
    stride = (lay.total_bytes + 255) // 256 * 256
    buf = torch.zeros(8 * stride, dtype=torch.uint8, device="cuda")
    for c in range(8):
        buf[c * stride:c * stride + lay.total_bytes].copy_(big)
    xs = torch.from_numpy(activations(8, k, 77)).cuda()
    ys = torch.empty((8, n), dtype=torch.float32, device="cuda")
    qg.gemv_batched(fmt, buf, stride, xs, ys, 8, n, k)
    y0 = qg.gemv(fmt, small, xs[3], 64, k, out_f32=True)
    torch.cuda.synchronize()
    assert torch.equal(ys[3, :64], y0), f"{fmt} batched"


@pytest.mark.parametrize("fmt", ["q3sb", "q4g32"])
def test_matrix_core_plans_on_7b_shapes_sampled_rows(fmt):
    """The matrix-core kernel's launch plans at 8 and 16 activation rows on the 7B-like
    shapes: 4 row tiles per workgroup (11008 x 4096, 12288 x 4096 and 14336 x 4096, grids
    of 344, 384 and 448 workgroups at 2), 6 (22016 x 4096: 688 at 2, 344 at 4, both over
    one round of workgroups), and one tile per workgroup (4096 x 11008: 256 tiles, K over
    six passes); the oracle recomputes sampled output rows."""
    for n, k in ((11008, 4096), (12288, 4096), (14336, 4096), (22016, 4096), (4096, 11008)):
        w = laplace_weights(n, k, 0.02, n + 3 * k, outlier_frac=0.001)
        wd = device_weights(fmt, w)
        rows = _sampled_rows(n, n + k)
        _, w_hat = oracle_decode(fmt, w[rows])
        for m in (8, 16):
            x = activations(m, k, m + n)
            y = qg.gemm(fmt, wd, torch.from_numpy(x).cuda(), n, k, out_f32=True)
            y_ref, bound = oracle_y(w_hat, x)
            torch.cuda.synchronize()
            assert_close(y.cpu().numpy()[:, rows], y_ref, bound, f"{fmt} m={m} {n}x{k}")


@pytest.mark.parametrize("fmt", FMTS)
def test_32_row_launch_equals_two_16_row_launches(fmt):
    """17-32 rows run as one launch of the matrix-core decode kernel with two 16-row blocks
    sharing each decoded fragment (on these shapes the cost estimate prefers it to the
    prefill tiles); each block's sums are formed as in a 16-row launch, so the output equals,
    bit for bit, that of separate launches on rows 0-15 and 16-m. Shapes: one tile per
    workgroup (4096 x 4096: 256 row tiles), the two-stage pipeline over 4 tiles per
    workgroup (11008 x 4096), K over several passes (70 x 28672), a ragged n (1001 x 1024)."""
    for n, k in ((1001, 1024), (4096, 4096), (11008, 4096), (70, 28672)):
        wd = device_weights(fmt, laplace_weights(n, k, 0.02, 3 * n + k))
        for m in (21, 32):
            x = torch.from_numpy(activations(m, k, m * k + n)).cuda()
            y = qg.gemm(fmt, wd, x, n, k, out_f32=True)
            y0 = qg.gemm(fmt, wd, x[:16].contiguous(), n, k, out_f32=True)
            y1 = qg.gemm(fmt, wd, x[16:].contiguous(), n, k, out_f32=True)
            torch.cuda.synchronize()
            assert torch.equal(y[:16], y0), f"{fmt} m={m} {n}x{k} rows 0-15"
            assert torch.equal(y[16:], y1), f"{fmt} m={m} {n}x{k} rows 16-{m - 1}"
