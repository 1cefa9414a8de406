"""GPU parity of the streaming kernel's launch plans at batch 1.

The single-row kernel has three plans: a one-shot plan for launches that fit two waves per
SIMD (every wave loads its four rows at once), the pipelined plan with fixed runs of row
batches per wave, and the pipelined plan with a shared batch queue per workgroup for large
launches with K in one wave. All three run the same per-row arithmetic and the same wave
reduction, so a row's output must be bit-identical whichever plan computes it, and within the
2e-3 * sum |W_hat x| tolerance of the oracle. Covered here: one-shot single launches against
queued strided batches of the same matrix, a ragged row count (rows past n re-read row n - 1
and are not stored), a grouped launch of two 11008 x 4096 matrices (the gate and up
projections of the 7B-like layer, queued) against single launches of each (fixed runs), and a
grouped pair of 4096^2 matrices (one-shot).
"""
import numpy as np
import pytest

import dequant_gemv_q4g32_amd as qg
from gpu_util import assert_close, device_weights, oracle_decode, oracle_y
from workloads import activations, laplace_weights

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FMTS = ["q4g32", "q2sb", "q3sb", "q5sb", "q6sb", "q4g16", "q4g64", "q4g128", "q4a32", "q4g32h",
        "q2sb_bf16", "q3sb_bf16", "q5sb_bf16", "q6sb_bf16", "q3g32", "q5g32", "q3sb_planes"]


def _rows(n, seed, count=24):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, n - 2, n - 1], rng.choice(n, size=count, replace=False)]))


def _check_rows(fmt, w, rows, x, y, what):
    _, w_hat = oracle_decode(fmt, w[rows])
    y_ref, bound = oracle_y(w_hat, x[None, :])
    assert_close(np.asarray(y, np.float64)[rows][None, :], y_ref, bound, what)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n", [4096, 4099])
def test_queued_batch_equals_one_shot_singles(fmt, n):
    """8 GEMVs of n x 4096 in one strided batch (16384+ rows: the queued plan) against each
    member alone (the one-shot plan), bit for bit, and sampled rows against the oracle."""
    k, count = 4096, 8
    w = laplace_weights(n, k, 0.02, 640 + n)
    wd = device_weights(fmt, w)
    lay = qg.device_layout(fmt, n, k)
    stride = (lay.total_bytes + 255) // 256 * 256
    buf = torch.zeros(count * stride, dtype=torch.uint8, device="cuda")
    for c in range(count):
        buf[c * stride:c * stride + lay.total_bytes].copy_(wd)
    xs = activations(count, k, 99 + n)
    xd = torch.from_numpy(xs).cuda()
    yb = torch.full((count, n + 3), 5.0, dtype=torch.float32, device="cuda")
    qg.gemv_batched(fmt, buf, stride, xd, yb[:, :n], count, n, k)
    torch.cuda.synchronize()
    assert torch.all(yb[:, n:] == 5.0).item(), "batched GEMV wrote past row n"
    rows = _rows(n, n)
    for c in range(count):
        ys = qg.gemv(fmt, wd, xd[c], n, k, out_f32=True)
        assert torch.equal(yb[c, :n], ys), f"{fmt} member {c}: queued and one-shot plans differ"
    for c in (0, 5):
        _check_rows(fmt, w, rows, xs[c], yb[c, :n].cpu().numpy(), f"{fmt} n={n} member {c}")


@pytest.mark.parametrize("fmt", ["q4g32", "q2sb", "q3sb", "q5sb", "q6sb", "q4a32", "q3g32", "q5g32"])
def test_grouped_gate_up_queued_equals_single_launches(fmt):
    """Gate and up (11008 x 4096 each, one shared activation) in one grouped launch, which takes
    the queued plan, against a single launch of each (fixed runs), bit for bit."""
    n, k = 11008, 4096
    ws = [laplace_weights(n, k, 0.02, 7100 + i) for i in range(2)]
    wds = [device_weights(fmt, w) for w in ws]
    x = activations(1, k, 808)
    xd = torch.from_numpy(x).cuda()
    outs = [torch.empty((1, n), dtype=torch.float32, device="cuda") for _ in range(2)]
    qg.gemm_grouped(fmt, wds, [xd, xd], [(n, k), (n, k)], outs=outs)
    torch.cuda.synchronize()
    rows = _rows(n, 3)
    for i in range(2):
        ys = qg.gemv(fmt, wds[i], xd[0], n, k, out_f32=True)
        assert torch.equal(outs[i][0], ys), f"{fmt} matrix {i}: grouped (queued) and single launch differ"
        _check_rows(fmt, ws[i], rows, x[0], ys.cpu().numpy(), f"{fmt} matrix {i}")


@pytest.mark.parametrize("fmt", ["q4g32", "q3sb", "q5sb", "q6sb"])
def test_grouped_pair_one_shot_equals_single_launches(fmt):
    """Two 4096^2 matrices in one grouped launch (one-shot plan) against single launches."""
    n, k = 4096, 4096
    ws = [laplace_weights(n, k, 0.02, 7300 + i) for i in range(2)]
    wds = [device_weights(fmt, w) for w in ws]
    xs = activations(2, k, 809)
    xd = torch.from_numpy(xs).cuda()
    outs = [torch.empty((1, n), dtype=torch.float32, device="cuda") for _ in range(2)]
    qg.gemm_grouped(fmt, wds, [xd[0:1], xd[1:2]], [(n, k), (n, k)], outs=outs)
    torch.cuda.synchronize()
    rows = _rows(n, 4)
    for i in range(2):
        ys = qg.gemv(fmt, wds[i], xd[i], n, k, out_f32=True)
        assert torch.equal(outs[i][0], ys), f"{fmt} matrix {i}: grouped and single launch differ"
        _check_rows(fmt, ws[i], rows, xs[i], ys.cpu().numpy(), f"{fmt} matrix {i}")
