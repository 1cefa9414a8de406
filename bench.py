#!/usr/bin/env python3
"""Benchmark: effective weight GB/s of batch-1 dequant GEMV on one MI355X.

Metric (DBHOO-CIM page, section 4.4: effective bandwidth = weight bytes / latency): the
algorithmic bytes of the packed weights (codes + every scale byte) divided by the GPU time,
reported as GB/s and as a fraction of the 8 TB/s HBM peak.

Workload (default): the 3-bit super-block matrix 4096 x 4096 (Laplace(0, 0.02) weights, fp16
N(0, 1) activations, batch 1). One step is one launch of G independent batch-1 GEMVs of that
shape (default G = 32, 230 MB of packed weights), each with its own matrix copy and its own
activation vector. Steps rotate over enough copies (>= 1.2 GB) that every step reads its
weights from HBM, not from the 256 MB last-level cache. The K timed steps are captured in one
HIP graph; after W eager warmup steps, one untimed replay (which uploads the graph) and 0.15 s
of back-to-back untimed replays (the clocks ramp under sustained load), the graph is replayed
between two synchronizes. A single 7.2 MB matrix per launch is also timed ("single_launch"),
and reported with the INT4 one under "batch1_one_matrix_per_launch": at ~1 us of streaming
it is bound by launch cadence, not HBM.

Beside the headline: the same steps launched eagerly on the stream ("stream_ms_per_step"),
the bytes of activations and outputs per launch (not counted in the metric), and the time of
the host quantizer (C++) for the headline matrix, as context.

"other_workloads" measures the remaining workloads the same way (HBM-resident rotation,
graph-timed): INT4 group-32 4096^2; the 7B-like layer set per super-block format (all seven
matrices in one grouped launch, and in the launches a decode step's data dependencies allow;
rotated over 32 copies, a 32-layer model's decode pass); the 70B-like layer set at batch 1,
2, 4, 8 and 16 (one launch per matrix, and one grouped launch); INT4 with groups of 16, 32,
64 and 128, the other format variants and act-order INT4 on the 70B-like set; the 8-bit
KV-cache codec on the 7B-like cache; and the 512-row prefill GEMM (TFLOP/s and fraction of
the 2.5 PFLOP/s dense fp16 MFMA peak), with 2048 rows as context.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "effective weight GB/s (and % of HBM peak) for batch-1 dequant GEMV"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="q3sb_gemv_4096")
    ap.add_argument("--group", type=int, default=32, help="independent batch-1 GEMVs per launch")
    ap.add_argument("--footprint-gb", type=float, default=1.2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-single", action="store_true", help="skip the one-matrix-per-launch timing")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (INT4 4096^2, layer sets, decode batches, prefill)")
    ap.add_argument("--profile-workload", default=None, metavar="NAME",
                    help="only run --steps rounds over the matrices of workload NAME, rotated over >= 1.2 GB "
                         "of copies, eagerly (for profiler runs; kv_cache_int8_7b_8192: rounds of the KV-cache "
                         "codec); prints no JSON line")
    ap.add_argument("--profile-plan", choices=("single", "group", "act_order"), default="single",
                    help="one launch per matrix, all matrices in one grouped launch, or one act-order "
                         "launch per matrix (a random column permutation per matrix)")
    ap.add_argument("--profile-fmt", default=None, help="weight format instead of the workload's")
    ap.add_argument("--profile-m", type=int, default=None, help="batch (activation rows) instead of the workload's")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 512 MiB device copy (the reference kernel for HBM counters)")
    return ap.parse_args()


SOURCES = ["dequant_gemv_q4g32_amd/csrc/gemv.hip", "dequant_gemv_q4g32_amd/csrc/mv.h",
           "dequant_gemv_q4g32_amd/csrc/units.h", "dequant_gemv_q4g32_amd/csrc/device_common.h",
           "dequant_gemv_q4g32_amd/csrc/layout.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the timed kernel from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by the same counter's reading for a
    plain copy of known size), or None if there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    fetch = float(kv["fetch_kib_per_dispatch"]) * 1024 * float(kv["copy_fetch_factor"])
    write = float(kv["write_kib_per_dispatch"]) * 1024 * float(kv["copy_write_factor"])
    return fetch + write


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(fmt, canonical, n, k, x, seconds):
    """The oracle as it stands (NumPy decode + fp64 matvec) on a bounded sample of rows of the
    same matrix, timed twice: on one thread, and on one thread per available core (at most 16)
    with each thread taking 64-row chunks in turn (NumPy releases the interpreter lock inside
    its array operations; BLAS is held to one thread per caller). Returns GB/s of packed
    weights processed; `value` is the all-core figure."""
    import threading

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import gemv as ogemv
    from oracle import int4
    from oracle import superblock as sb

    chunk = 64
    row_bytes = canonical.size // n

    def rows(r0, r1):
        if fmt == "q4g32":
            codes = canonical[: n * k // 2].reshape(n, k // 2)[r0:r1]
            scales = canonical[n * k // 2:].view(np.float32).reshape(n, k // 32)[r0:r1]
            w_hat = int4.decode(codes, scales, k)
        else:
            w_hat = sb.decode(fmt, canonical.reshape(n, k // 256, -1)[r0:r1])
        ogemv.gemv(w_hat, x)

    def run(threads):
        lock = threading.Lock()
        state = {"next": 0, "done": 0}
        t0 = time.perf_counter()

        def worker():
            while time.perf_counter() - t0 < seconds:
                with lock:
                    r0 = state["next"] % n
                    state["next"] = r0 + chunk
                r1 = min(n, r0 + chunk)
                rows(r0, r1)
                with lock:
                    state["done"] += r1 - r0

        ts = [threading.Thread(target=worker) for _ in range(threads)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        dt = time.perf_counter() - t0
        return state["done"], dt

    affinity = len(os.sched_getaffinity(0))
    threads = max(1, min(16, affinity))
    with threadpool_limits(1):
        done1, dt1 = run(1)
        done, dt = run(threads)
    one = round(done1 * row_bytes / dt1 / 1e9, 4)
    return {"value": round(done * row_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "one_thread_value": one, "cpu_model": _cpu_model(), "sched_getaffinity_cpus": affinity,
            "sample": f"{done} rows ({done / n:.2f} passes) of the {n}x{k} {fmt} matrix on {threads} threads in "
                      f"{dt:.1f} s, and {done1} rows on one thread in {dt1:.1f} s: NumPy decode of the canonical "
                      f"encoding + fp64 matvec"}


MFMA_F16_PEAK_TFLOPS = 2500.0
# the 7B-like KV cache: K and V of 32 layers x 8192 tokens, 8 KV heads x 128 per row
KV_WORKLOAD = "kv_cache_int8_7b_8192"
KV_ROWS, KV_COLS = 2 * 32 * 8192, 8 * 128


WARM_S = 0.15     # sustained load before a timed replay: the clocks drop within a second of idle


def _warm(replay, seconds=WARM_S):
    """Run replay() back to back for `seconds`: after the idle of host-side set-up the GPU
    clocks take tens of milliseconds of load to ramp (a 512-row prefill launch measures 93 us
    right after a second of idle and 80 us after 50 ms of load)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        replay()
        torch.cuda.synchronize()


def _graph_time_us(fn, rounds, reps=3):
    """Median over reps of the per-round time of `rounds` calls of fn(i), captured in one graph
    and replayed after WARM_S seconds of back-to-back replays."""
    import torch
    fn(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(rounds):
            fn(i)
    _warm(g.replay)
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / rounds)
    del g
    return sorted(times)[len(times) // 2]


def build_set(qg, fmt, canon_shapes, m, dev, plan, footprint_gb=1.2, min_copies=2):
    """Device buffers for passes over a set of matrices (batch m), with the weights rotated over
    enough copies that every round reads them from HBM. `plan` lists the launches of a round:
    ("group", [i, ...]) is one grouped launch of those matrices (any shapes), ("batched",
    [i, ...]) one strided batched launch of consecutive same-shape matrices (m = 1), ("single",
    [i]) one qg_gemm (qg_gemv at m = 1), ("act_order", [i]) one qg_gemm_act_order with a random
    column permutation. At least min_copies copies (a model's layer count). Returns (algorithmic
    bytes per round, rnd) where rnd(r) issues round r."""
    import numpy as np
    import torch
    from workloads import activations
    lays = [qg.device_layout(fmt, n, k) for _, n, k in canon_shapes]
    strides = [(l.total_bytes + 255) // 256 * 256 for l in lays]
    set_bytes = sum(strides)
    alg = sum(l.algorithmic_bytes for l in lays)
    copies = max(min_copies, int(np.ceil(footprint_gb * 1e9 / set_bytes)))
    buf = torch.empty(copies * set_bytes, dtype=torch.uint8, device=dev)
    offs = np.concatenate([[0], np.cumsum(strides)[:-1]]).astype(np.int64)
    for j, (canon, n, k) in enumerate(canon_shapes):
        one = torch.from_numpy(qg.to_device_layout(fmt, canon, n, k)).to(dev)
        for c in range(copies):
            o = c * set_bytes + int(offs[j])
            buf[o:o + lays[j].total_bytes].copy_(one)
        del one
    shapes = [(n, k) for _, n, k in canon_shapes]
    launches = []
    for kind, idx in plan:
        if kind == "batched":
            n, k = shapes[idx[0]]
            X = torch.from_numpy(activations(len(idx), k, 11 + idx[0])).to(dev)
            Y = torch.empty((len(idx), n), dtype=torch.float16, device=dev)
        else:
            X = [torch.from_numpy(activations(m, shapes[i][1], 11 + i)).to(dev) for i in idx]
            Y = [torch.empty((m, shapes[i][0]), dtype=torch.float16, device=dev) for i in idx]
        P = None
        if kind == "act_order":
            P = torch.from_numpy(np.random.default_rng(idx[0]).permutation(shapes[idx[0]][1]).astype(np.int32)).to(dev)
        launches.append((kind, idx, X, Y, P))

    def rnd(r):
        base = (r % copies) * set_bytes
        for kind, idx, X, Y, P in launches:
            if kind == "act_order":
                (i,) = idx
                qg.gemm_act_order(fmt, buf[base + int(offs[i]):], X[0], P, shapes[i][0], shapes[i][1], out=Y[0])
            elif kind == "batched":
                n, k = shapes[idx[0]]
                qg.gemv_batched(fmt, buf[base + int(offs[idx[0]]):], strides[idx[0]], X, Y, len(idx), n, k)
            elif kind == "group":
                qg.gemm_grouped(fmt, [buf[base + int(offs[i]):] for i in idx], X, [shapes[i] for i in idx], outs=Y)
            else:
                (i,) = idx
                n, k = shapes[i]
                if m == 1:
                    qg.gemv(fmt, buf[base + int(offs[i]):], X[0][0], n, k, out=Y[0][0])
                else:
                    qg.gemm(fmt, buf[base + int(offs[i]):], X[0], n, k, out=Y[0])

    return alg, rnd


def measure_set(qg, fmt, canon_shapes, m, dev, plan, footprint_gb=1.2, rounds=24, min_copies=2):
    """build_set, then the graph-timed microseconds per round: (algorithmic bytes, us)."""
    import torch
    alg, rnd = build_set(qg, fmt, canon_shapes, m, dev, plan, footprint_gb, min_copies)
    us = _graph_time_us(rnd, rounds)
    del rnd
    torch.cuda.empty_cache()
    return alg, us


def _rate(alg, us):
    return {"GBps": round(alg / us / 1e3, 1), "frac": round(alg / us / 1e3 / HBM_PEAK_GBPS, 4), "us": round(us, 2)}


def extra_configs(qg, dev):
    """The other workloads on this one GPU: INT4 group-32 4096^2 at batch 1, the 7B-like layer
    set (q/k/v/o, gate/up, down) per super-block format, the 70B-like set at batch 1, 2, 4, 8
    and 16, and the 512-row prefill GEMM (with 2048 rows as context)."""
    from workloads import WORKLOADS
    out = {}
    # INT4 group-32 4096 x 4096, batch 1: 32 per launch like the headline, and one per launch
    wl = WORKLOADS["q4g32_gemv_4096"]
    canon = qg.quantize("q4g32", wl.weights(0))
    alg, us = measure_set(qg, "q4g32", [(canon, 4096, 4096)] * 32, 1, dev, [("batched", list(range(32)))], rounds=16)
    alg1, us1 = measure_set(qg, "q4g32", [(canon, 4096, 4096)], 1, dev, [("single", [0])], rounds=200)
    out["q4g32_gemv_4096"] = {"GBps_32_per_launch": round(alg / us / 1e3, 1), "frac": round(alg / us / 1e3 / HBM_PEAK_GBPS, 4),
                              "GBps_single_launch": round(alg1 / us1 / 1e3, 1), "us_single_launch": round(us1, 2)}
    log(f"[bench] q4g32 4096^2: {out['q4g32_gemv_4096']}")
    # context only: the same 32 GEMVs of 4096 x 4096 with dense fp16 weights (33.5 MB each, the
    # traffic the quantized formats avoid), one torch bmm per launch over contiguous operands
    import torch
    sets = 2
    wd = torch.randn((sets, 32, 4096, 4096), dtype=torch.float16, device=dev)
    xd = torch.randn((32, 4096, 1), dtype=torch.float16, device=dev)
    yd = torch.empty((32, 4096, 1), dtype=torch.float16, device=dev)
    for i in range(4):
        torch.bmm(wd[i % sets], xd, out=yd)             # (eager: a library GEMM stays out of graphs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(20):
        torch.bmm(wd[i % sets], xd, out=yd)
    e1.record()
    torch.cuda.synchronize()
    us_d = e0.elapsed_time(e1) * 1e3 / 20
    dense_bytes = 32 * 4096 * 4096 * 2
    out["dense_fp16_gemv_4096_x32"] = {"us": round(us_d, 2), "weight_GBps": round(dense_bytes / us_d / 1e3, 1)}
    log(f"[bench] dense fp16 context, 32 x 4096^2 GEMV per launch: {out['dense_fp16_gemv_4096_x32']}")
    del wd, xd, yd
    torch.cuda.empty_cache()
    # 7B-like layer set, batch 1, each format (the four share one set of fp32 weights). Matrices
    # 0-3 are q, k, v, o; 4, 5 gate, up; 6 down. "one_launch": all seven in one grouped launch;
    # "decode_order": the launches a decode step can issue given its data dependencies
    # ({q, k, v} share x; o waits for attention; {gate, up} share x; down waits for both).
    # The weights rotate over 32 copies of the set at least: one round is one layer of a
    # 32-layer 7B-class model, so 32 rounds are one token's decode pass.
    wl = WORKLOADS["q3sb_7b_layer_set"]
    w7 = [wl.weights(i) for i in range(len(wl.shapes))]
    for fmt in ("q2sb", "q3sb", "q5sb", "q6sb"):
        cs = [(qg.quantize(fmt, w), w.shape[0], w.shape[1]) for w in w7]
        alg, us = measure_set(qg, fmt, cs, 1, dev, [("group", list(range(7)))], rounds=32, min_copies=32)
        alg2, us2 = measure_set(qg, fmt, cs, 1, dev, [("group", [0, 1, 2]), ("single", [3]), ("group", [4, 5]),
                                                      ("single", [6])], rounds=32, min_copies=32)
        out[f"{fmt}_7b_layer_set"] = {**_rate(alg, us), "bytes_per_set": alg,
                                      "decode_order": _rate(alg2, us2)}
        log(f"[bench] {fmt} 7B layer set: {out[f'{fmt}_7b_layer_set']}")
    del w7
    # context: the read probe alone over the same launch pattern (q3sb byte counts), i.e. the
    # rate at which launches of these sizes can stream at all: the decode-order rounds (qkv,
    # o, gate+up, down as 4 probe launches per round) and one 4096^2 matrix per launch
    import torch
    lay4, lay11, layd = (qg.device_layout("q3sb", n, k) for n, k in ((4096, 4096), (11008, 4096), (4096, 11008)))
    sizes = [3 * lay4.algorithmic_bytes, lay4.algorithmic_bytes, 2 * lay11.algorithmic_bytes, layd.algorithmic_bytes]
    sizes = [(b + 15) // 16 * 16 for b in sizes]
    span = (sum(sizes) + 255) // 256 * 256
    copies = int(1.2e9 // span) + 1
    pbuf = torch.zeros(copies * span, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    offs = [0, sizes[0], sizes[0] + sizes[1], sizes[0] + sizes[1] + sizes[2]]

    def probe_round(r):
        base = (r % copies) * span
        for o, b in zip(offs, sizes):
            qg.read_probe(pbuf[base + o:], b, sink)
    us_p = _graph_time_us(probe_round, 32)
    one = (lay4.algorithmic_bytes + 255) // 256 * 256
    n1 = int(1.2e9 // one)
    us_1 = _graph_time_us(lambda r: qg.read_probe(pbuf[(r % n1) * one:], lay4.algorithmic_bytes // 16 * 16, sink), 200)
    out["read_probe_launch_patterns_context"] = {
        "decode_order_7b_q3sb": _rate(sum(sizes), us_p),
        "one_4096sq_q3sb_matrix": _rate(lay4.algorithmic_bytes, us_1)}
    log(f"[bench] read probe over the same launch patterns: {out['read_probe_launch_patterns_context']}")
    del pbuf
    torch.cuda.empty_cache()
    # 70B-like layer set at batch 1, 2, 4, 8, 16, 32 (q3sb and q5sb share the fp32 weights): one launch
    # per matrix (the matrices depend on each other in a decode step), and all three in one
    # grouped launch (up to batch 8)
    wl = WORKLOADS["q3sb_70b_layer_set_m1"]
    w70 = [wl.weights(i) for i in range(len(wl.shapes))]
    for fmt in ("q3sb", "q5sb"):
        cs = [(qg.quantize(fmt, w), w.shape[0], w.shape[1]) for w in w70]
        for m in (1, 2, 4, 8, 16, 32):
            alg, us = measure_set(qg, fmt, cs, m, dev, [("single", [0]), ("single", [1]), ("single", [2])], rounds=12)
            flops = 2 * m * sum(n * k for _, n, k in cs)
            out[f"{fmt}_70b_layer_set_m{m}"] = {**_rate(alg, us), "TFLOPs": round(flops / us / 1e6, 2)}
            if m <= 8:      # grouped launches take up to 8 activation rows
                alg2, us2 = measure_set(qg, fmt, cs, m, dev, [("group", [0, 1, 2])], rounds=12)
                out[f"{fmt}_70b_layer_set_m{m}"]["one_launch"] = _rate(alg2, us2)
            log(f"[bench] {fmt} 70B layer set m={m}: {out[f'{fmt}_70b_layer_set_m{m}']}")
        del cs
    del w70
    # INT4 group sizes (16, 32, 64, 128), asymmetric groups of 32, fp16-scale groups of 32, the
    # bf16 super-scale variants of q3sb and q5sb, and plain group-wise 3- and 5-bit codes on
    # the 70B-like set at batch 1, one launch per matrix
    w70 = [WORKLOADS["q3sb_70b_layer_set_m1"].weights(i) for i in range(3)]
    for fmt in ("q4g16", "q4g32", "q4g64", "q4g128", "q4a32", "q4g32h", "q3sb_bf16", "q5sb_bf16", "q3g32", "q5g32"):
        cs = [(qg.quantize(fmt, w), w.shape[0], w.shape[1]) for w in w70]
        alg, us = measure_set(qg, fmt, cs, 1, dev, [("single", [0]), ("single", [1]), ("single", [2])], rounds=12)
        out[f"{fmt}_70b_layer_set_m1"] = {**_rate(alg, us), "bytes_per_set": alg}
        log(f"[bench] {fmt} 70B layer set m=1: {out[f'{fmt}_70b_layer_set_m1']}")
        del cs
    del w70
    # act-order INT4 (GPTQ-style column permutation, the gather fused into the kernel) on the
    # 70B-like set at batch 1, against the same launches without the permutation
    cs = [(qg.quantize("q4g32", w), w.shape[0], w.shape[1]) for w in
          (WORKLOADS["q3sb_70b_layer_set_m1"].weights(i) for i in range(3))]
    alg, us = measure_set(qg, "q4g32", cs, 1, dev, [("act_order", [0]), ("act_order", [1]), ("act_order", [2])], rounds=12)
    alg2, us2 = measure_set(qg, "q4g32", cs, 1, dev, [("single", [0]), ("single", [1]), ("single", [2])], rounds=12)
    out["q4g32_70b_layer_set_act_order_m1"] = {**_rate(alg, us), "without_permutation": _rate(alg2, us2)}
    log(f"[bench] q4g32 70B layer set, act-order, m=1: {out['q4g32_70b_layer_set_act_order_m1']}")
    del cs
    # 8-bit KV-cache codec on the 7B-like cache (32 layers x K and V x 8 KV heads x 128, 8192
    # tokens = 536,870,912 elements): bytes moved = 2 (fp16) + 1.0625 (codes and scales) per
    # element; and the per-token append of a decode step (64 rows of 1024)
    import torch
    from workloads import activations
    rows, cols = KV_ROWS, KV_COLS
    x = torch.empty((rows, cols), dtype=torch.float16, device=dev)
    x.copy_(torch.from_numpy(activations(1024, cols, 3)).to(dev).repeat(rows // 1024, 1))
    codes = torch.empty((rows, cols), dtype=torch.int8, device=dev)
    scales = torch.empty((rows, cols // 32), dtype=torch.float16, device=dev)
    moved = rows * cols * 3.0625
    us_q = _graph_time_us(lambda i: qg.kv_quantize(x, codes, scales), 4)
    us_d = _graph_time_us(lambda i: qg.kv_dequantize(codes, scales, out=x), 4)
    xa, ca, sa = x[:64], codes[:64], scales[:64]
    us_a = _graph_time_us(lambda i: qg.kv_quantize(xa, ca, sa), 200)
    out["kv_cache_int8_7b_8192"] = {"quantize_GBps": round(moved / us_q / 1e3, 1), "quantize_us": round(us_q, 1),
                                    "dequantize_GBps": round(moved / us_d / 1e3, 1), "dequantize_us": round(us_d, 1),
                                    "frac": round(max(moved / us_q, moved / us_d) / 1e3 / HBM_PEAK_GBPS, 4),
                                    "append_one_token_us": round(us_a, 2)}
    log(f"[bench] KV cache int8 codec: {out['kv_cache_int8_7b_8192']}")
    del x, codes, scales
    torch.cuda.empty_cache()
    # prefill: 512 x 4096 activations times 11008 x 4096 weights (MFMA bound), and 2048 rows
    # of activations as context
    for fmt in ("q4g32", "q5sb"):
        wl = WORKLOADS[f"{fmt}_prefill_512"]
        n, k = wl.shapes[0]
        canon = qg.quantize(fmt, wl.weights(0))
        for m in (512, 2048):
            alg, us = measure_set(qg, fmt, [(canon, n, k)], m, dev, [("single", [0])], rounds=10)
            tf = 2 * m * n * k / us / 1e6
            key = f"{fmt}_prefill_512" if m == 512 else f"{fmt}_prefill_{m}_context"
            out[key] = {"TFLOPs": round(tf, 1), "mfma_frac_of_fp16_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                        "us": round(us, 2), "weight_GBps": round(alg / us / 1e3, 1)}
            log(f"[bench] {fmt} prefill {m}: {out[key]}")
    # context only: the same 512 x 4096 x 11008 product with dense fp16 weights through torch's
    # GEMM (the vendor library; timed eagerly after the clocks ramp, library GEMMs stay out of
    # graphs), the work the low-bit formats add a decode to
    import torch
    n, k = WORKLOADS["q4g32_prefill_512"].shapes[0]
    xa = torch.randn((512, k), dtype=torch.float16, device=dev)
    wts = [torch.randn((k, n), dtype=torch.float16, device=dev) for _ in range(8)]   # 8 x 90 MB, past the LLC
    ya = torch.empty((512, n), dtype=torch.float16, device=dev)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < WARM_S:
        torch.matmul(xa, wts[0], out=ya)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(40):
        torch.matmul(xa, wts[i % 8], out=ya)
    e1.record()
    torch.cuda.synchronize()
    us_m = e0.elapsed_time(e1) * 1e3 / 40
    tf = 2 * 512 * n * k / us_m / 1e6
    out["dense_fp16_prefill_512_context"] = {"TFLOPs": round(tf, 1), "mfma_frac_of_fp16_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                                             "us": round(us_m, 2)}
    log(f"[bench] dense fp16 prefill context: {out['dense_fp16_prefill_512_context']}")
    del xa, wts, ya
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the dequant GEMV path is "
                                   "single-GPU (row sharding across GPUs is a design note only)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import dequant_gemv_q4g32_amd as qg
    from workloads import WORKLOADS

    if args.profile_workload == KV_WORKLOAD:
        # the 8-bit KV-cache codec on the 7B-like cache: --steps rounds of quantize + dequantize
        from workloads import activations
        dev = torch.device("cuda:0")
        rows, cols = KV_ROWS, KV_COLS
        x = torch.empty((rows, cols), dtype=torch.float16, device=dev)
        x.copy_(torch.from_numpy(activations(1024, cols, 3)).to(dev).repeat(rows // 1024, 1))
        codes = torch.empty((rows, cols), dtype=torch.int8, device=dev)
        scales = torch.empty((rows, cols // 32), dtype=torch.float16, device=dev)

        def one_kv():
            qg.kv_quantize(x, codes, scales)
            qg.kv_dequantize(codes, scales, out=x)
        _warm(one_kv)
        for r in range(args.steps):
            one_kv()
        torch.cuda.synchronize()
        log(f"[bench] profiled {KV_WORKLOAD}: {args.steps} rounds of quantize + dequantize, {rows} x {cols} fp16")
        return
    if args.profile_workload:
        wl = WORKLOADS[args.profile_workload]
        m = args.profile_m or wl.m
        fmt = args.profile_fmt or wl.fmt
        cs = [(qg.quantize(fmt, wl.weights(i)), n, k) for i, (n, k) in enumerate(wl.shapes)]
        idx = list(range(len(cs)))
        plan = [("group", idx)] if args.profile_plan == "group" else [(args.profile_plan, [i]) for i in idx]
        alg, rnd = build_set(qg, fmt, cs, m, torch.device("cuda:0"), plan, args.footprint_gb)
        state = {"r": 0}

        def one():
            rnd(state["r"])
            state["r"] += 1
        _warm(one)          # rounds before the last --steps: clock ramp, not measured
        warm_rounds = state["r"]
        for r in range(args.steps):
            one()
        torch.cuda.synchronize()
        log(f"[bench] profiled {args.profile_workload}: {args.steps} rounds of {len(plan)} launches after "
            f"{warm_rounds} warm-up rounds, {fmt} m={m}, shapes {list(wl.shapes)}, {alg} algorithmic bytes per round")
        return

    wl = WORKLOADS[args.workload]
    fmt = wl.fmt
    n, k = wl.shapes[0]
    dev = torch.device("cuda:0")
    log(f"[bench] {args.workload}: {fmt} {n}x{k}, {args.group} GEMVs per launch")

    w = wl.weights(0)
    # the host quantizer (C++, synchronous; offline in a deployment, timed here as context)
    tq = []
    for _ in range(3):
        t0 = time.perf_counter()
        canonical = qg.quantize(fmt, w)
        tq.append(time.perf_counter() - t0)
    host_quantize = {"s_per_matrix": round(sorted(tq)[1], 4),
                     "Mweights_per_s": round(n * k / sorted(tq)[1] / 1e6, 1),
                     "what": f"qg_quantize of the {n}x{k} fp32 matrix to {fmt} records, one host thread"}
    lay = qg.device_layout(fmt, n, k)
    alg = lay.algorithmic_bytes
    stride = (lay.total_bytes + 255) // 256 * 256
    one = torch.from_numpy(qg.to_device_layout(fmt, canonical, n, k)).to(dev)

    G = args.group
    sets = max(3, int(np.ceil(args.footprint_gb * 1e9 / (G * stride))))
    copies = sets * G
    buf = torch.empty(copies * stride, dtype=torch.uint8, device=dev)
    for c in range(copies):
        buf[c * stride:c * stride + lay.total_bytes].copy_(one)
    xs = torch.from_numpy(wl.x(0, m=copies)).to(dev)
    ys = torch.empty((copies, n), dtype=torch.float16, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] {copies} copies x {stride / 1e6:.2f} MB = {copies * stride / 1e9:.2f} GB resident")

    def step(i):
        s = i % sets
        qg.gemv_batched(fmt, buf[s * G * stride:], stride, xs[s * G:], ys[s * G:], G, n, k)

    # The K timed steps are captured in one HIP graph (so that host launch overhead cannot
    # leave the GPU idle between 50 us steps). After the W warmup steps the graph is replayed
    # once untimed (its first replay uploads it) and back to back for WARM_S seconds, then
    # timed between two synchronizes.
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            step(args.warmup + i)
    graph.replay()
    torch.cuda.synchronize()
    _warm(graph.replay)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    del graph
    gbps = G * alg / (ms * 1e-3) / 1e9
    log(f"[bench] grouped: {ms * 1e3:.2f} us per launch, {gbps:.0f} GB/s")
    # the same steps launched eagerly, back to back on the stream (host launch overhead can
    # leave gaps between launches)
    ns = min(args.steps, 200)
    ev0.record()
    for i in range(ns):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    ms_stream = ev0.elapsed_time(ev1) / ns

    # check the timed outputs of one set against a single-matrix launch (same kernels)
    ref = qg.gemv(fmt, one, xs[0], n, k)
    torch.cuda.synchronize()
    assert torch.equal(ref, ys[0]), "grouped output differs from single launch"

    # read ceiling over the same resident buffer
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    span = sets * G * stride // 3 // 16 * 16
    for i in range(3):
        qg.read_probe(buf[(i % 3) * span:], span, sink)
    torch.cuda.synchronize()
    ev0.record()
    reps = 12
    for i in range(reps):
        qg.read_probe(buf[(i % 3) * span:], span, sink)
    ev1.record()
    torch.cuda.synchronize()
    ceiling = span / (ev0.elapsed_time(ev1) / reps * 1e-3) / 1e9
    log(f"[bench] read ceiling ({span / 1e6:.0f} MB per launch): {ceiling:.0f} GB/s")

    single = None
    if not args.no_single:
        iters = 400
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(iters):
                qg.gemv(fmt, buf[(i % copies) * stride:], xs[i % copies], n, k, out=ys[i % copies])
        _warm(g.replay)
        ev0.record()
        for i in range(iters):
            qg.gemv(fmt, buf[(i % copies) * stride:], xs[i % copies], n, k, out=ys[i % copies])
        ev1.record()
        torch.cuda.synchronize()
        us_stream = ev0.elapsed_time(ev1) / iters * 1e3
        _warm(g.replay, 0.05)
        ev0.record()
        g.replay()
        ev1.record()
        torch.cuda.synchronize()
        us_graph = ev0.elapsed_time(ev1) / iters * 1e3
        single = {"us_per_gemv_stream": round(us_stream, 3), "GBps_stream": round(alg / us_stream / 1e3, 1),
                  "us_per_gemv_graph": round(us_graph, 3), "GBps_graph": round(alg / us_graph / 1e3, 1)}
        log(f"[bench] single launch: stream {us_stream:.2f} us, graph {us_graph:.2f} us per GEMV")

    if args.calibrate_copy:
        # a plain device copy of known size: its FETCH_SIZE / WRITE_SIZE readings give the
        # factors that turn those counters into bytes
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] ran 5 copies of 512 MiB for counter calibration")

    extra = None
    if not args.no_extra:
        extra = extra_configs(qg, dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host ...")
        cpu = cpu_baseline(fmt, canonical, n, k, wl.x(0)[0], args.cpu_seconds)
        log(f"[bench] oracle: {cpu['value']} GB/s ({cpu['sample']})")

    traffic = measured_traffic(args.workload)
    # one matrix per launch at batch 1 (the headline packs 32 independent GEMVs into a launch),
    # and the 7B-like layer set in the launches a decode step's dependencies allow
    per_matrix = {f"{args.workload}": single}
    decode_order = None
    if extra:
        q4 = extra["q4g32_gemv_4096"]
        per_matrix["q4g32_gemv_4096"] = {"us_per_gemv_graph": q4["us_single_launch"], "GBps_graph": q4["GBps_single_launch"]}
        decode_order = {f: extra[f"{f}_7b_layer_set"]["decode_order"]["frac"] for f in ("q2sb", "q3sb", "q5sb", "q6sb")}
    for v in per_matrix.values():
        if v:
            v["frac_graph"] = round(v["GBps_graph"] / HBM_PEAK_GBPS, 4)
    out = {
        "metric": METRIC, "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16xfp16->fp32", "data": "synthetic",
        "config": {"workload": f"{args.workload}: {fmt} {n}x{k}, batch 1, {G} independent matrices per launch",
                   "fmt": fmt, "n": n, "k": k, "batch": 1, "matrices_per_launch": G,
                   "algorithmic_bytes_per_matrix": alg, "resident_GB": round(copies * stride / 1e9, 3)},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic},
        "headline_kind": f"multi-matrix throughput: {G} independent batch-1 GEMVs per launch",
        "batch1_one_matrix_per_launch": per_matrix,
        "layer_set_7b_decode_order_frac": decode_order,
        "algorithmic_bytes_per_launch": G * alg,
        "activation_and_output_bytes_per_launch": G * (k + n) * 2,
        "stream_ms_per_step": round(ms_stream, 5),
        "stream_GBps": round(G * alg / (ms_stream * 1e-3) / 1e9, 1),
        "host_quantize": host_quantize,
        "read_ceiling_GBps": round(ceiling, 1),
        "frac_of_read_ceiling": round(gbps / ceiling, 4),
        "single_launch": single,
        "cpu_baseline": cpu,
        "other_workloads": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
