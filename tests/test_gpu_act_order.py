"""GPU parity tests for act-order weights (qg_gemm_act_order: the activation gather by the
stored column permutation, fused into the streaming kernel), against the oracle.

Bar: every output within 2e-3 * sum_k |X[i,k] W_eff[r,k]| of the oracle's W_eff X (the
stored columns scattered back to their original positions, oracle/actorder.py), and equal
bit for bit to qg_gemm on the gathered activations X[:, perm] (the same kernel arithmetic).
Covers every format, K over 1..5 waves, ragged q4g32 K, m in {1, 2, 3, 4, 8}, strided X,
a permutation entry outside [0, k) (reads 0), and a full-size 4096^2 matrix on sampled rows.
"""
import numpy as np
import pytest

import dequant_gemv_q4g32_amd as qg
from gpu_util import assert_close, device_weights, oracle_decode, oracle_y
from oracle import actorder
from workloads import activations, laplace_weights

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FMTS = ["q4g32", "q2sb", "q3sb", "q5sb", "q6sb", "q4g16", "q4g128", "q4a32", "q4g32h", "q3sb_bf16", "q5sb_bf16", "q3g32", "q5g32"]
# the three forms by rows x k: two LDS copies (natural and stored-column order) up to 128 KB,
# one natural-order copy with per-lane gathers up to 128 KB (k = 8192 at 4 and 8 rows), none
# beyond (k = 8448 at 8 rows: per-lane gathers from global memory)
SHAPES = [(37, 512), (300, 4352), (9, 8192), (9, 8448)]


def _case(fmt, n, k, seed):
    rng = np.random.default_rng(seed)
    w = laplace_weights(n, k, 0.02, seed)
    perm = rng.permutation(k)
    stored = actorder.stored_matrix(w, perm).astype(np.float32)
    _, w_hat_s = oracle_decode(fmt, stored)
    return perm, device_weights(fmt, stored), actorder.effective_weights(w_hat_s, perm)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", SHAPES)
def test_act_order_matches_oracle_and_gathered_gemm(fmt, n, k):
    perm, wd, w_eff = _case(fmt, n, k, 3 * n + k)
    pd = torch.from_numpy(perm.astype(np.int32)).cuda()
    for m in (1, 2, 3, 4, 8):
        x = activations(m, k, 11 * m + k)
        X = torch.from_numpy(x).cuda()
        y = qg.gemm_act_order(fmt, wd, X, pd, n, k, out_f32=True)
        # the same streaming kernel on the gathered activations (qg_gemm takes it up to 4 rows),
        # launched on the same row chunks (rows past 128 KB of activations run in halves, ...)
        Xg = X[:, torch.from_numpy(perm).cuda()].contiguous()
        ref = torch.empty_like(y)
        mc = m
        while mc > 1 and mc * k * 2 > 128 * 1024:
            mc = (mc + 1) // 2
        for r in range(0, m, mc):
            qg.gemm_grouped(fmt, [wd], [Xg[r:r + mc]], [(n, k)], outs=[ref[r:r + mc]])
        torch.cuda.synchronize()
        y_ref, bound = oracle_y(w_eff, x)
        assert_close(y.cpu().numpy(), y_ref, bound, f"{fmt} m={m} {n}x{k}")
        assert torch.equal(y, ref), f"{fmt} m={m}: act-order != gathered streaming launch"


def test_act_order_vector_form_ragged_q4g32_and_strided():
    n, k = 70, 4128                      # k % 64 == 32: the last unit is half a unit
    perm, wd, w_eff = _case("q4g32", n, k, 77)
    pd = torch.from_numpy(perm.astype(np.int32)).cuda()
    x = activations(1, k, 5)
    y = qg.gemm_act_order("q4g32", wd, torch.from_numpy(x[0]).cuda(), pd, n, k, out_f32=True)
    torch.cuda.synchronize()
    y_ref, bound = oracle_y(w_eff, x)
    assert_close(y.cpu().numpy()[None, :], y_ref, bound, "ragged vector")
    # strided X (ldx = k + 40) and Y (ldy = n + 3), 3 rows
    xm = activations(3, k, 6)
    xbuf = torch.zeros((3, k + 40), dtype=torch.float16, device="cuda")
    xbuf[:, :k] = torch.from_numpy(xm).cuda()
    ybuf = torch.full((3, n + 3), 7.0, dtype=torch.float32, device="cuda")
    qg.gemm_act_order("q4g32", wd, xbuf[:, :k], pd, n, k, out=ybuf[:, :n])
    torch.cuda.synchronize()
    yb = ybuf.cpu().numpy()
    assert np.all(yb[:, n:] == 7.0)
    y_ref, bound = oracle_y(w_eff, xm)
    assert_close(yb[:, :n], y_ref, bound, "strided")


def test_act_order_index_out_of_range_reads_zero():
    """A permutation entry outside [0, k) reads an activation of 0 (and nothing outside X)."""
    fmt, n, k = "q3sb", 40, 512
    perm, wd, w_eff = _case(fmt, n, k, 99)
    bad = perm.astype(np.int32).copy()
    bad[17] = k + 1000
    bad[300] = -5
    x = activations(2, k, 8)
    y = qg.gemm_act_order(fmt, wd, torch.from_numpy(x).cuda(), torch.from_numpy(bad).cuda(), n, k, out_f32=True)
    xz = x.copy()
    xz[:, perm[17]] = 0
    xz[:, perm[300]] = 0
    torch.cuda.synchronize()
    y_ref, bound = oracle_y(w_eff, xz)
    assert_close(y.cpu().numpy(), y_ref, bound, "out-of-range entries")


def test_act_order_full_size_sampled_rows():
    n = k = 4096
    fmt = "q4g32"
    rng = np.random.default_rng(4096)
    w = laplace_weights(n, k, 0.02, 4096, outlier_frac=0.001)
    perm = rng.permutation(k)
    stored = actorder.stored_matrix(w, perm).astype(np.float32)
    wd = device_weights(fmt, stored)
    x = activations(1, k, 12)
    y = qg.gemm_act_order(fmt, wd, torch.from_numpy(x[0]).cuda(), torch.from_numpy(perm.astype(np.int32)).cuda(), n, k)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 30, replace=False)]))
    _, w_hat_s = oracle_decode(fmt, stored[rows])
    y_ref, bound = oracle_y(actorder.effective_weights(w_hat_s, perm), x)
    assert_close(y.cpu().float().numpy()[None, rows], y_ref, bound, "full size")
