"""GPU parity tests for the prefill dequant GEMM (m > 16: fp16 tiles in LDS, MFMA), against
the oracle.

Bar: every output Y[i, r] within 2e-3 * sum_k |X[i,k] W_hat[r,k]|. The fp16 dequantized
weights carry at most two fp16 roundings (about 1e-3 of |w_hat|), inside that bound.
The kernel tiles Y in 256 activation rows by 64 weight rows, by 96 where those tiles fill
the rounds of workgroups on the CUs better, or in 128 by 32 where 256 x 64 tiles would leave
CUs without a workgroup. Covers all three tile shapes (the small shapes below and 512 x 4099 take 128 x 32
tiles, except where qg_gemm's cost estimate runs the rows as 32-row matrix-core decode
launches instead: 130 x 4352 at 64 rows, and in some formats 130 x 4352 at 128 rows and
300 x 1024 at 64; the wide shapes 256 x 64; 300 x 10003 and the full-size workloads 256 x 96), m
below, at and above one M tile and ragged across several, n not a multiple of either weight
tile, K over one and many steps, ragged q4g32 K, strided X and Y, fp16 and fp32 output, and
the full-size 512 x 11008 x 4096 prefill workloads on sampled weight rows.
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
SHAPES = [(37, 256), (300, 1024), (130, 4352)]
MS = [9, 64, 128, 200]


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
def test_prefill_matches_oracle(fmt, n, k):
    w = laplace_weights(n, k, 0.02, 13 * n + k, outlier_frac=0.001)
    _, w_hat = oracle_decode(fmt, w)
    wd = device_weights(fmt, w)
    for m in MS:
        x = activations(m, k, 3 * m + k)
        y_ref, bound = oracle_y(w_hat, x)
        assert_close(_run(fmt, wd, x, n, k, True), y_ref, bound, f"{fmt} m={m} {n}x{k} f32")
        if m == 200:
            assert_close(_run(fmt, wd, x, n, k, False), y_ref, bound, f"{fmt} m={m} {n}x{k} f16")


@pytest.mark.parametrize("fmt", FMTS)
def test_prefill_strided(fmt):
    n, k, m = 150, 512, 70
    w = laplace_weights(n, k, 0.02, 4242)
    _, w_hat = oracle_decode(fmt, w)
    x = activations(m, k, 11)
    y_ref, bound = oracle_y(w_hat, x)
    y = _run(fmt, device_weights(fmt, w), x, n, k, True, ldx=k + 40, ldy=n + 3)
    assert_close(y, y_ref, bound, f"{fmt} strided")


def test_prefill_q4g32_ragged_k():
    for n, k in ((40, 96), (130, 4128)):
        w = laplace_weights(n, k, 0.02, k + 5)
        _, w_hat = oracle_decode("q4g32", w)
        x = activations(33, k, k)
        y_ref, bound = oracle_y(w_hat, x)
        assert_close(_run("q4g32", device_weights("q4g32", w), x, n, k, True), y_ref, bound, f"q4g32 {n}x{k}")


@pytest.mark.parametrize("fmt", FMTS)
def test_prefill_one_hot_rows(fmt):
    """X rows are unit vectors e_c: output row i is column c_i of W_hat, which pins where every
    decoded weight lands in the LDS tile and in the MFMA operands."""
    n, k = 136, 256
    w = laplace_weights(n, k, 0.02, 77)
    _, w_hat = oracle_decode(fmt, w)
    m = 40
    cols = (np.arange(m) * 37 + 3) % k
    x = np.zeros((m, k), np.float16)
    x[np.arange(m), cols] = 1.0
    y = _run(fmt, device_weights(fmt, w), x, n, k, True)
    want = w_hat[:, cols].T
    # one fp16 rounding of the dequantized weight (and of step / p for symmetric formats); the
    # absolute term covers the fp32 rounding of an asymmetric weight whose two parts cancel
    tol = 1.2e-3 * np.abs(want) + 1e-6
    assert np.all(np.abs(y - want) <= tol), np.argwhere(np.abs(y - want) > tol)[:5]


def _prefill_cases():
    return [name for name, wl in WORKLOADS.items() if wl.m > 8]


@pytest.mark.parametrize("name", _prefill_cases())
def test_full_size_prefill_sampled_rows(name):
    """The full prefill shape (512 x 4096 activations, 11008 x 4096 weights) in the launch
    configuration the library uses for it; the oracle recomputes sampled weight rows (output
    columns) for all 512 activation rows."""
    wl = WORKLOADS[name]
    n, k = wl.shapes[0]
    w = wl.weights(0)
    x = wl.x(0)
    wd = device_weights(wl.fmt, w)
    y = qg.gemm(wl.fmt, wd, torch.from_numpy(x).cuda(), n, k)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 127, 128, n - 1], rng.choice(n, 28, replace=False)]))
    _, w_hat = oracle_decode(wl.fmt, w[rows])
    y_ref, bound = oracle_y(w_hat, x)
    torch.cuda.synchronize()
    assert_close(y.cpu().float().numpy()[:, rows], y_ref, bound, name)


@pytest.mark.parametrize("fmt", ["q4g32", "q3sb", "q5sb", "q6sb", "q2sb", "q4a32", "q3g32"])
@pytest.mark.parametrize("m,n,k", [(300, 16384 - 3, 256), (520, 8256 - 3, 512), (500, 4096 + 3, 512),
                                   (300, 10000 + 3, 256)])
def test_prefill_tile_shapes_several_m_tiles(fmt, m, n, k):
    """256 x 64 tiles (the first two shapes: 512 and 387 of them) over two or three M tiles,
    128 x 32 tiles (the third: 2 x 65 tiles of 256 x 64 would leave CUs idle) over four, and
    256 x 96 tiles (the fourth: 314 tiles of 256 x 64, 210 of 256 x 96), each with a ragged
    last M tile and ragged n; sampled weight rows against the oracle."""
    w = laplace_weights(n, k, 0.02, 77 + m, outlier_frac=0.001)
    wd = device_weights(fmt, w)
    x = activations(m, k, 5 + m)
    y = _run(fmt, wd, x, n, k, True)
    rng = np.random.default_rng(m)
    rows = np.unique(np.concatenate([[0, 31, 32, 63, 64, 95, 96, n - 1], rng.choice(n, size=40, replace=False)]))
    _, w_hat = oracle_decode(fmt, w[rows])
    y_ref, bound = oracle_y(w_hat, x)
    assert_close(y[:, rows], y_ref, bound, f"{fmt} {m}x{n}x{k}")
