"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This module holds no quantization, packing or GEMV arithmetic: only random draws with
the shapes and value distributions of the workloads, so that the oracle and the HIP
path can be fed identical inputs without sharing any of the method's code.

Distributions (stand-ins for trained layers, which are not available here):
  * weights: zero-centred Laplace(0, b), drawn in fp64 and rounded through fp16 to
    fp32, mimicking an fp16 checkpoint ("二三五六" page, section 2.1 notes that weight
    distributions are roughly zero-centred Laplacian);
  * optional outliers: an exact count round(frac * n * k) of positions, drawn without
    replacement, multiplied by a factor (the DBHOO-CIM page, section 2.1, motivates
    group-32 scales by such outliers);
  * activations: fp16 standard normal.

Weights and activations of one workload come from separate children of one
SeedSequence, so that changing the activation shape never changes the weights.
"""
from __future__ import annotations

import dataclasses
from typing import List, Tuple

import numpy as np

BASE_SEED = 20261200


def _children(seed: int, n: int) -> List[np.random.Generator]:
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(n)]


def laplace_weights(n: int, k: int, b: float, seed: int, outlier_frac: float = 0.0,
                    outlier_mult: float = 20.0) -> np.ndarray:
    """fp32 [n, k] weights: Laplace(0, b) rounded through fp16, optional outliers."""
    rng_w, rng_o = _children(seed, 2)
    w = rng_w.laplace(0.0, b, size=(n, k))
    if outlier_frac > 0.0 and n * k > 0:
        cnt = int(round(outlier_frac * n * k))
        idx = rng_o.choice(n * k, size=cnt, replace=False)
        w.reshape(-1)[idx] *= outlier_mult
    return w.astype(np.float16).astype(np.float32)


def activations(m: int, k: int, seed: int) -> np.ndarray:
    """fp16 [m, k] standard-normal activations."""
    (rng,) = _children(seed + 7_000_000, 1)
    return rng.standard_normal(size=(m, k)).astype(np.float16)


def uniform_codes(count: int, bits: int, seed: int) -> np.ndarray:
    """uint8 [count] uniform integers in [0, 2**bits) for bitstream round trips."""
    (rng,) = _children(seed, 1)
    return rng.integers(0, 1 << bits, size=count, dtype=np.uint8)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named synthetic workload: a format, a list of weight shapes and a batch."""
    name: str
    fmt: str
    shapes: Tuple[Tuple[int, int], ...]   # (n = out_features, k = in_features)
    b: float                              # Laplace scale parameter
    m: int = 1                            # activation rows (batch)
    outlier_frac: float = 0.0
    seed: int = BASE_SEED

    def weights(self, i: int) -> np.ndarray:
        n, k = self.shapes[i]
        return laplace_weights(n, k, self.b, self.seed + 100 * i, self.outlier_frac)

    def x(self, i: int, m: int | None = None) -> np.ndarray:
        n, k = self.shapes[i]
        return activations(self.m if m is None else m, k, self.seed + 100 * i)

    @property
    def weight_count(self) -> int:
        return sum(n * k for n, k in self.shapes)


LAYER_7B = ((4096, 4096),) * 4 + ((11008, 4096),) * 2 + ((4096, 11008),)
LAYER_70B = ((8192, 8192), (28672, 8192), (8192, 28672))

WORKLOADS = {
    # INT4 group-32, 4096 x 4096 with 0.1 % outliers x20, batch 1
    "q4g32_gemv_4096": Workload("q4g32_gemv_4096", "q4g32", ((4096, 4096),), 0.02, 1, 0.001, BASE_SEED + 1),
    # 3-bit super-block, 4096 x 4096, batch 1
    "q3sb_gemv_4096": Workload("q3sb_gemv_4096", "q3sb", ((4096, 4096),), 0.02, 1, 0.0, BASE_SEED + 2),
}
for _f in ("q2sb", "q3sb", "q5sb", "q6sb"):
    WORKLOADS[f"{_f}_7b_layer_set"] = Workload(f"{_f}_7b_layer_set", _f, LAYER_7B, 0.02, 1, 0.0, BASE_SEED + 3)
for _f in ("q3sb", "q5sb"):
    for _m in (1, 2, 4, 8):
        WORKLOADS[f"{_f}_70b_layer_set_m{_m}"] = Workload(f"{_f}_70b_layer_set_m{_m}", _f, LAYER_70B, 0.015, _m,
                                                          0.0, BASE_SEED + 4)
for _f in ("q4g32", "q5sb"):
    WORKLOADS[f"{_f}_prefill_512"] = Workload(f"{_f}_prefill_512", _f, ((11008, 4096),), 0.02, 512, 0.0,
                                              BASE_SEED + 5)
