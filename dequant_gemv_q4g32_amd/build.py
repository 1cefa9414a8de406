"""Build libqgemv.so in-tree with hipcc for gfx950.

Host code (quantizers, layouts) is compiled as plain C++ with -ffp-contract=off so that no
multiply-add is fused in the quantizers' integer decisions. Device code is compiled for
gfx950 only, with packed fp32 instructions disabled and also with -ffp-contract=off: every
fused multiply-add in the kernels is written out (fmaf, v_dot2), so that a kernel's
arithmetic, and a row's result, does not depend on which instantiation computes it (the
compiler would otherwise pick which product of a*b + c*d to fuse from the surrounding code).

Usage: python dequant_gemv_q4g32_amd/build.py  (a plain script: it must not import the package,
whose import loads the library it builds).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqgemv.so")

HOST_SOURCES = ["host.cpp"]
DEVICE_SOURCES = ["gemv.hip", "prefill.hip", "skinny.hip", "kvcache.hip"] + sorted(
    f for f in os.listdir(CSRC) if f.startswith("mv_") and f.endswith(".hip"))   # streaming launchers per format
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libqgemv")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return res


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    common = ["-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{ROOT}/include"]
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run([hipcc, "-x", "c++", "-O2", "-ffp-contract=off", *common, "-c", os.path.join(CSRC, src), "-o", obj],
             verbose)
        objs.append(obj)
    device = []
    for src in DEVICE_SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(BUILD, src + ".o")
        device.append([hipcc, f"--offload-arch={ARCH}", "-O3", "-ffp-contract=off", *common,
                       "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                       "-c", path, "-o", obj])
        objs.append(obj)
    # the device sources compile independently: one compiler process each
    with ThreadPoolExecutor(max_workers=max(1, min(len(device), os.cpu_count() or 1, 8))) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd in device]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp, "-lpthread"], verbose)
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized(verbose: bool = False) -> str:
    """The host code alone (quantizers, bitstreams, layouts) as a CPU shared library built by g++
    with AddressSanitizer and UndefinedBehaviorSanitizer, aborting on the first report. It is
    loaded through QGEMV_HOST_ONLY_LIBRARY by the host tests (see the package docstring); a
    process that loads it must preload the ASan runtime (g++ -print-file-name=libasan.so)."""
    gxx = shutil.which("g++")
    if not gxx:
        raise RuntimeError("g++ not found")
    os.makedirs(BUILD, exist_ok=True)
    out = os.path.join(BUILD, "libqgemv_host_san.so")
    tmp = out + ".tmp"
    _run([gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fPIC", "-shared",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", f"-I{ROOT}/include",
          os.path.join(CSRC, "host.cpp"), "-o", tmp, "-lpthread"], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
