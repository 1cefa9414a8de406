"""GPU parity tests for the grouped launch (several matrices of different shapes in one
launch), against the oracle and against the single-matrix entry points.

Bar: every output within 2e-3 * sum_k |X[i,k] W_hat[r,k]|, as for qg_gemm. For m <= 4 the
grouped launch runs the same streaming kernel with the same split of K as qg_gemm, so its
outputs must also equal qg_gemm's bit for bit. Covers mixed K (one wave to several waves
along K, and two passes over K with eight activation rows), ragged n, a shared activation
(q/k/v style), matrices with n == 0 and k == 0 inside a group, fp16 and fp32 output, and
the full-size 7B-like layer set (4 x 4096^2, 2 x 11008 x 4096, 4096 x 11008) in one
launch on sampled output rows.
"""
import numpy as np
import pytest

import dequant_gemv_q4g32_amd as qg
from gpu_util import assert_close, device_weights, oracle_decode, oracle_y
from workloads import WORKLOADS, activations, laplace_weights

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FMTS = ["q4g32", "q2sb", "q3sb", "q5sb", "q6sb", "q4g16", "q4g128", "q4a32", "q4g32h", "q3sb_bf16", "q5sb_bf16", "q3g32", "q5g32"]
# K over 1, 2, 5 and 7 waves; ragged n; (7, 28672) takes two passes over K at m = 8
SHAPES = [(37, 512), (300, 4352), (9, 8192), (130, 1024), (7, 28672), (64, 4352)]


def _mats(fmt, seed):
    out = []
    for i, (n, k) in enumerate(SHAPES):
        w = laplace_weights(n, k, 0.02, seed + 31 * i, outlier_frac=0.001)
        out.append((n, k, oracle_decode(fmt, w)[1], device_weights(fmt, w)))
    return out


def _run_group(fmt, mats, xs, out_f32):
    """outs via one grouped launch, each in a guarded buffer wider than n."""
    dt = torch.float32 if out_f32 else torch.float16
    m = xs[0].shape[0]
    bufs = [torch.full((m, n + 5), 3.0, dtype=dt, device="cuda") for n, _, _, _ in mats]
    qg.gemm_grouped(fmt, [wd for _, _, _, wd in mats], xs, [(n, k) for n, k, _, _ in mats],
                    outs=[b[:, :n] for b, (n, _, _, _) in zip(bufs, mats)])
    torch.cuda.synchronize()
    res = []
    for b, (n, _, _, _) in zip(bufs, mats):
        yb = b.cpu().float().numpy()
        assert np.all(yb[:, n:] == 3.0), "grouped GEMM wrote outside Y[:, :n]"
        res.append(yb[:, :n])
    return res


@pytest.mark.parametrize("fmt", FMTS)
def test_grouped_matches_oracle_and_single_launches(fmt):
    mats = _mats(fmt, 900)
    for m in (1, 2, 3, 4, 8):
        xs_np = [activations(m, k, 7 * m + k + i) for i, (_, k, _, _) in enumerate(mats)]
        # q/k/v style: matrices 1 and 5 (both K = 4352) read the same activation tensor
        xs = [torch.from_numpy(x).cuda() for x in xs_np]
        xs[5] = xs[1]
        xs_np[5] = xs_np[1]
        for out_f32 in ((True, False) if m in (1, 4) else (True,)):
            ys = _run_group(fmt, mats, xs, out_f32)
            for i, ((n, k, w_hat, wd), y) in enumerate(zip(mats, ys)):
                y_ref, bound = oracle_y(w_hat, xs_np[i])
                assert_close(y, y_ref, bound, f"{fmt} m={m} matrix {i} {n}x{k} f32={out_f32}")
                if m <= 4:
                    single = qg.gemm(fmt, wd, xs[i], n, k, out_f32=out_f32)
                    torch.cuda.synchronize()
                    assert np.array_equal(single.cpu().float().numpy(), y), f"{fmt} m={m} matrix {i}: grouped != qg_gemm"


def test_grouped_vector_form_and_degenerate_members():
    """m = 1 with 1-D activations and outputs; a member with n == 0 is skipped and one with
    k == 0 gets zeros, while the others are computed."""
    fmt = "q3sb"
    mats = _mats(fmt, 4000)[:3]
    x = [torch.from_numpy(activations(1, k, k)[0]).cuda() for _, k, _, _ in mats]
    empty_w = torch.zeros(256, dtype=torch.uint8, device="cuda")
    y_k0 = torch.full((11,), 5.0, dtype=torch.float16, device="cuda")
    ws = [mats[0][3], empty_w, mats[1][3], empty_w, mats[2][3]]
    xs = [x[0], x[0][:0], x[1], x[0], x[2]]
    shapes = [(mats[0][0], mats[0][1]), (0, 256), (mats[1][0], mats[1][1]), (11, 0), (mats[2][0], mats[2][1])]
    outs = qg.gemm_grouped(fmt, ws, xs, shapes)
    outs[3] = y_k0
    qg.gemm_grouped(fmt, ws, xs, shapes, outs=outs)
    torch.cuda.synchronize()
    assert np.all(y_k0.cpu().numpy() == 0)
    for j, i in ((0, 0), (2, 1), (4, 2)):
        n, k, w_hat, _ = mats[i]
        y_ref, bound = oracle_y(w_hat, x[i].cpu().numpy()[None, :])
        assert_close(outs[j].cpu().float().numpy()[None, :], y_ref, bound, f"member {j}")


def test_grouped_full_size_7b_layer_set_sampled_rows():
    """The 7B-like layer set of seven matrices at batch 1 in one launch (the launch shape the
    library uses for it); the oracle recomputes sampled rows of every matrix."""
    wl = WORKLOADS["q3sb_7b_layer_set"]
    ws_np = [wl.weights(i) for i in range(len(wl.shapes))]
    wds = [device_weights(wl.fmt, w) for w in ws_np]
    xs_np = [activations(1, w.shape[1], 50 + i)[0] for i, w in enumerate(ws_np)]
    ys = qg.gemm_grouped(wl.fmt, wds, [torch.from_numpy(x).cuda() for x in xs_np], [w.shape for w in ws_np])
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    for i, (w, x, y) in enumerate(zip(ws_np, xs_np, ys)):
        n = w.shape[0]
        rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 14, replace=False)]))
        _, w_hat = oracle_decode(wl.fmt, w[rows])
        y_ref, bound = oracle_y(w_hat, x[None, :])
        assert_close(y.cpu().float().numpy()[None, rows], y_ref, bound, f"7B set matrix {i}")
