"""GPU parity across input magnitudes: the tolerance of the dequantize-and-multiply is scale-free
(|y - y_ref| <= 2e-3 * sum_k |W_hat[r,k] X[m,k]| per output), so it must hold for small layers
and small activations as well as for the Laplace(0, 0.02) / N(0, 1) inputs of the workloads.

Every format, on every kernel qg_gemm routes to: the GEMV (1 row), the streaming kernel
(3 rows), the matrix-core decode kernel (8 rows) and the prefill kernel (24 rows), with
  * weight scales b in {0.02, 2e-3, 2e-4} (Laplace(0, b));
  * activation scales {1, 1e-2, 1e-3, 1e-4} times N(0, 1), and mixed magnitudes: each
    element times 10^u with u uniform in [-4, 0], and each activation row at its own scale.
fp32 outputs everywhere; fp16 outputs too where the tolerance of the smallest outputs stays
well above half an fp16 subnormal unit (2^-25), which no fp16 result can beat.

The matrix-core paths round each decoded weight to fp16. The symmetric INT4 and 3-bit formats
take their step (or group scale) through fp16 first, which keeps full precision down to steps
of 2^-14; the weight scales here keep the steps above it (b = 2e-4 gives 3-bit steps near
2e-4 and INT4 group-of-16 scales near 8e-5).
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
W_SCALES = [0.02, 2e-3, 2e-4]
A_SCALES = [1.0, 1e-2, 1e-3, 1e-4, "mixed"]
MS = [1, 3, 8, 24]          # GEMV, streaming, matrix-core decode, prefill
N, K = 100, 4352            # two prefill row tiles (ragged), 68 units: more than one wave along K


def _x(m, scale, seed):
    base = activations(m, K, seed).astype(np.float64)
    if scale == "mixed":
        rng = np.random.default_rng(seed)
        elem = 10.0 ** rng.uniform(-4.0, 0.0, size=base.shape)
        rows = 10.0 ** -(np.arange(m) % 5)[:, None].astype(np.float64)
        return (base * elem * rows).astype(np.float16), 1e-4 * 1e-4
    return (base * scale).astype(np.float16), scale


def _gemm(fmt, wd, x, out_f32):
    m = x.shape[0]
    y = torch.full((m, N), 3.0, dtype=torch.float32 if out_f32 else torch.float16, device="cuda")
    qg.gemm(fmt, wd, torch.from_numpy(x).cuda(), N, K, out=y)
    torch.cuda.synchronize()
    return y.cpu().float().numpy()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("b", W_SCALES)
def test_parity_across_magnitudes(fmt, b):
    w = laplace_weights(N, K, b, 9100 + int(-np.log10(b) * 10), outlier_frac=0.001)
    _, w_hat = oracle_decode(fmt, w)
    wd = device_weights(fmt, w)
    for ai, a in enumerate(A_SCALES):
        for m in MS:
            x, a_small = _x(m, a, 300 * ai + m)
            y_ref, bound = oracle_y(w_hat, x)
            what = f"{fmt} b={b} x~{a} m={m}"
            assert_close(_gemm(fmt, wd, x, True), y_ref, bound, what + " f32")
            if b * a_small >= 2e-6:
                assert_close(_gemm(fmt, wd, x, False), y_ref, bound, what + " f16")
