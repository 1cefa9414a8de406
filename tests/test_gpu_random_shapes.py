"""Seeded random shapes through qg_gemm and qg_gemm_act_order: every format, activation rows
from 1 to 2100 (the streaming kernel, the matrix-core small-M kernel and the three prefill
tile shapes, each with ragged m and n), K up to 4096.

Reference: the fp32 product of the activations with W_hat decoded on the device by
qg_dequantize (whose decode is bit-exact against the oracle, tests/test_gpu_gemv.py), in
plain PyTorch fp32; bar: every output within 2e-3 * sum_k |x w_hat| (plus 1e-6)."""
import numpy as np
import pytest

import dequant_gemv_q4g32_amd as qg
from workloads import activations, laplace_weights

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MS = [1, 2, 3, 4, 5, 8, 13, 16, 17, 40, 100, 256, 257, 300, 511, 512, 700, 1024, 1500, 2100]


def _cases(count, seed):
    rng = np.random.default_rng(seed)
    fmts = list(qg.FORMATS)
    out = []
    for c in range(count):
        fmt = fmts[c % len(fmts)]
        k = 256 * int(rng.integers(1, 17))
        n = int(rng.integers(1, 6001))
        m = int(rng.choice(MS))
        out.append((fmt, m, n, k, int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("fmt,m,n,k,seed", _cases(34, 2024))
def test_random_shape_matches_fp32_product(fmt, m, n, k, seed):
    dev = torch.device("cuda")
    w = laplace_weights(n, k, 0.02, seed)
    wd = torch.from_numpy(qg.to_device_layout(fmt, qg.quantize(fmt, w), n, k)).to(dev)
    X = torch.from_numpy(activations(m, k, seed + 1)).to(dev)
    w_hat, _ = qg.dequantize(fmt, wd, n, k, codes=False)
    Xf = X.float()
    y = qg.gemm(fmt, wd, X, n, k, out_f32=True)
    ref = Xf @ w_hat.t()
    bound = Xf.abs() @ w_hat.abs().t()
    torch.cuda.synchronize()
    assert bool(((y - ref).abs() <= 2e-3 * bound + 1e-6).all()), f"{fmt} m={m} n={n} k={k}"
    if m <= 8:
        perm = torch.from_numpy(np.random.default_rng(seed).permutation(k).astype(np.int32)).to(dev)
        ya = qg.gemm_act_order(fmt, wd, X, perm, n, k, out_f32=True)
        Xp = Xf[:, perm.long()]
        ref_a = Xp @ w_hat.t()
        bound_a = Xp.abs() @ w_hat.abs().t()
        torch.cuda.synchronize()
        assert bool(((ya - ref_a).abs() <= 2e-3 * bound_a + 1e-6).all()), f"act-order {fmt} m={m} n={n} k={k}"
