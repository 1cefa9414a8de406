"""Every device entry point allocates nothing and synchronizes nothing, so its launches can be
captured in a HIP graph. One graph holds a GEMV, GEMMs with 3, 8 and 40 activation rows (the
streaming, matrix-core decode and prefill kernels), a grouped launch and the KV-cache codec;
it is replayed several times, with eager launches of the same kernels on other inputs
between the replays, and every replay's outputs must equal the eager results bit for bit."""
import numpy as np
import pytest

import dequant_gemv_q4g32_amd as qg
from gpu_util import device_weights
from workloads import activations, laplace_weights

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["q3sb", "q4g32", "q5sb"])
def test_graph_replays_equal_eager(fmt):
    n, k = 1000, 1024
    wd = device_weights(fmt, laplace_weights(n, k, 0.02, 31))
    wd2 = device_weights(fmt, laplace_weights(n, k, 0.02, 32))
    xs = {m: torch.from_numpy(activations(m, k, 40 + m)).cuda() for m in (1, 3, 8, 40)}
    kv_x = torch.from_numpy(activations(64, 256, 7)).cuda()

    def run(w, outs):
        qg.gemv(fmt, w, xs[1][0], n, k, out=outs["gemv"])
        for m in (3, 8, 40):
            qg.gemm(fmt, w, xs[m], n, k, out=outs[f"gemm{m}"])
        qg.gemm_grouped(fmt, [w, w], [xs[3], xs[3]], [(n, k), (n, k)], outs=[outs["g0"], outs["g1"]])
        qg.kv_quantize(kv_x, outs["codes"], outs["scales"])
        qg.kv_dequantize(outs["codes"], outs["scales"], out=outs["kv"])

    def buffers():
        b = {"gemv": torch.empty(n, dtype=torch.float16, device="cuda")}
        for m in (3, 8, 40):
            b[f"gemm{m}"] = torch.empty((m, n), dtype=torch.float16, device="cuda")
        b["g0"] = torch.empty((3, n), dtype=torch.float16, device="cuda")
        b["g1"] = torch.empty((3, n), dtype=torch.float16, device="cuda")
        b["codes"] = torch.empty((64, 256), dtype=torch.int8, device="cuda")
        b["scales"] = torch.empty((64, 8), dtype=torch.float16, device="cuda")
        b["kv"] = torch.empty((64, 256), dtype=torch.float16, device="cuda")
        return b

    eager = buffers()
    run(wd, eager)
    torch.cuda.synchronize()
    ref = {key: v.clone() for key, v in eager.items()}

    graphed = buffers()
    run(wd, graphed)                    # one eager call before capture (no allocation inside)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(wd, graphed)
    other = buffers()
    for rep in range(4):
        for v in graphed.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        run(wd2, other)                 # eager work on other weights between the replays
        torch.cuda.synchronize()
        for key, v in graphed.items():
            assert torch.equal(v, ref[key]), f"{fmt} replay {rep}: {key} differs from the eager result"
    assert not torch.equal(other["gemm8"], ref["gemm8"])   # the eager work really used other weights
