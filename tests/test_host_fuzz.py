"""Property test of the host quantizers: for random shapes, scales and value mixes (zeros,
tiny and large magnitudes, single-sign blocks), every format's canonical bytes from the C++
host library equal the oracle's (two independent implementations of the same rules), and
the device layout round-trips. CPU only."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import dequant_gemv_q4g32_amd as qg
from test_host_library import FMTS, oracle_canonical


@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(fmt=st.sampled_from(FMTS), rows=st.integers(1, 5), blocks=st.integers(1, 3),
       seed=st.integers(0, 2**31 - 1), scale=st.sampled_from([1e-6, 1e-3, 0.02, 1.0, 300.0]),
       mix=st.sampled_from(["laplace", "sparse", "positive", "negative", "constant"]))
def test_quantizer_bytes_match_oracle(fmt, rows, blocks, seed, scale, mix):
    k = blocks * 256
    rng = np.random.default_rng(seed)
    w = rng.laplace(0.0, scale, size=(rows, k))
    if mix == "sparse":
        w *= rng.random((rows, k)) < 0.05
    elif mix == "positive":
        w = np.abs(w)
    elif mix == "negative":
        w = -np.abs(w)
    elif mix == "constant":
        w[:] = scale
    w = w.astype(np.float32)
    got = qg.quantize(fmt, w)
    assert np.array_equal(got, oracle_canonical(fmt, w))
    dev = qg.to_device_layout(fmt, got, rows, k)
    assert np.array_equal(qg.from_device_layout(fmt, dev, rows, k), got)
