"""Python binding of libqgemv (ctypes). Argument marshalling only: every step of the
quantize / pack / dequant-GEMV path runs in the C++ host library or in the HIP kernels.

PyTorch supplies device memory and streams: device arguments are torch tensors on a ROCm
device, and work is enqueued on torch's current stream unless ``stream`` is given.
Importing this module fails if the shared library has not been built
(``python dequant_gemv_q4g32_amd/build.py``); there is no fallback implementation.

QGEMV_HOST_ONLY_LIBRARY=<path> loads a build of the host code alone instead (the sanitizer
build of ``build.build_host_sanitized``): only the host functions are bound then, and every
device entry point is absent, so calling one raises instead of running anywhere else.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_ONLY_LIB = os.environ.get("QGEMV_HOST_ONLY_LIBRARY")
LIB_PATH = HOST_ONLY_LIB or os.path.join(_HERE, "libqgemv.so")
# exported by the host code (host.cpp); everything else is device code
HOST_FUNCTIONS = ("qg_abi_version", "qg_strerror", "qg_canonical_bytes", "qg_device_layout",
                  "qg_packed_bytes", "qg_pack_bits", "qg_unpack_bits", "qg_quantize", "qg_to_device_layout",
                  "qg_from_device_layout")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "qgemv.h")

FORMATS = {"q2sb": 2, "q3sb": 3, "q4g32": 4, "q5sb": 5, "q6sb": 6, "q4g16": 7, "q4g64": 8, "q4g128": 9,
           "q4a32": 10, "q4g32h": 11,
           "q2sb_bf16": 12, "q3sb_bf16": 13, "q5sb_bf16": 15, "q6sb_bf16": 16, "q3g32": 17, "q5g32": 18,
           "q3sb_planes": 14}
GROUPWISE_FORMATS = ("q3g32", "q5g32")   # plain group-wise codes, fp32 scale and min per 32
Q4_GROUPS = {"q4g16": 16, "q4g32": 32, "q4g64": 64, "q4g128": 128}   # symmetric INT4 group sizes
SUPERBLOCK_FORMATS = ("q2sb", "q3sb", "q5sb", "q6sb", "q2sb_bf16", "q3sb_bf16", "q5sb_bf16", "q6sb_bf16",
                      "q3sb_planes")
K_MULTIPLE = {"q4g32": 32, "q2sb": 256, "q3sb": 256, "q5sb": 256, "q6sb": 256, "q4g16": 64, "q4g64": 64, "q4g128": 128,
              "q4a32": 64, "q4g32h": 64, "q2sb_bf16": 256, "q3sb_bf16": 256, "q5sb_bf16": 256,
              "q6sb_bf16": 256, "q3g32": 64, "q5g32": 64,
              "q3sb_planes": 256}


class QGError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = f"{what}: {_lib.qg_strerror(status).decode()} (status {status})"
        if status == -7:
            msg += f"; HIP: {_lib.qg_last_hip_error().decode()}"
        super().__init__(msg)


class Layout(ctypes.Structure):
    _fields_ = [("total_bytes", ctypes.c_int64), ("algorithmic_bytes", ctypes.c_int64),
                ("nplanes", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("plane_offset", ctypes.c_int64 * 4), ("plane_row_bytes", ctypes.c_int64 * 4)]


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime under the same soname as ROCm's. Loading torch first
    # makes libqgemv bind to that one runtime; loading libqgemv first would map a second HIP
    # and HSA runtime into the process, which then finds no device, and torch's streams and
    # device pointers would mean nothing to it anyway.
    if not HOST_ONLY_LIB:
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python dequant_gemv_q4g32_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    sig = {
        "qg_abi_version": ([], i32),
        "qg_strerror": ([i32], ctypes.c_char_p),
        "qg_last_hip_error": ([], ctypes.c_char_p),
        "qg_canonical_bytes": ([i32, i64, i64, ctypes.POINTER(i64)], i32),
        "qg_device_layout": ([i32, i64, i64, ctypes.POINTER(Layout)], i32),
        "qg_packed_bytes": ([i32, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)], i32),
        "qg_pack_bits": ([i32, vp, i64, vp], i32),
        "qg_unpack_bits": ([i32, vp, i64, vp], i32),
        "qg_quantize": ([i32, vp, i64, i64, i64, vp], i32),
        "qg_to_device_layout": ([i32, vp, i64, i64, vp], i32),
        "qg_from_device_layout": ([i32, vp, i64, i64, vp], i32),
        "qg_gemv": ([i32, vp, vp, vp, i32, i64, i64, vp], i32),
        "qg_gemv_batched": ([i32, vp, i64, vp, i64, vp, i64, i32, i64, i64, i64, vp], i32),
        "qg_gemm": ([i32, vp, vp, i64, vp, i64, i32, i64, i64, i64, vp], i32),
        "qg_gemm_grouped": ([i32, i32, vp, vp, vp, vp, vp, vp, vp, i64, i32, vp], i32),
        "qg_gemm_act_order": ([i32, vp, vp, i64, vp, vp, i64, i32, i64, i64, i64, vp], i32),
        "qg_kv_quantize": ([vp, i64, i64, i64, vp, vp, vp], i32),
        "qg_kv_dequantize": ([vp, vp, i64, i64, vp, i64, vp], i32),
        "qg_dequantize": ([i32, vp, vp, vp, i64, i64, vp], i32),
        "qg_read_probe": ([vp, i64, vp, vp], i32),
    }
    for f in FORMATS:
        sig[f"quantize_{f}"] = ([vp, i64, i64, i64, vp], i32)
        sig[f"dequant_gemv_{f}"] = ([vp, vp, vp, i64, i64, vp], i32)
        sig[f"dequant_gemm_{f}"] = ([vp, vp, i64, vp, i64, i64, i64, i64, vp], i32)
        sig[f"dequantize_{f}"] = ([vp, vp, vp, i64, i64, vp], i32)
    for name, (args, res) in sig.items():
        if HOST_ONLY_LIB and not (name in HOST_FUNCTIONS or name.startswith("quantize_")):
            continue
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if lib.qg_abi_version() != 1:
        raise ImportError("libqgemv ABI version mismatch")
    return lib


_lib = _load()
lib = _lib


def declared_functions() -> list:
    """Names of the functions include/qgemv.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def _check(status: int, what: str) -> None:
    if status != 0:
        raise QGError(status, what)


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        return FORMATS[fmt]
    return int(fmt)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ---------------------------------------------------------------- host --------------------

def canonical_bytes(fmt, n: int, k: int) -> int:
    out = ctypes.c_int64()
    _check(_lib.qg_canonical_bytes(_fmt(fmt), n, k, ctypes.byref(out)), "qg_canonical_bytes")
    return out.value


def device_layout(fmt, n: int, k: int) -> Layout:
    out = Layout()
    _check(_lib.qg_device_layout(_fmt(fmt), n, k, ctypes.byref(out)), "qg_device_layout")
    return out


def pack_bits(bits: int, codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty((codes.size * bits + 7) // 8, np.uint8)
    _check(_lib.qg_pack_bits(bits, _ptr(codes), codes.size, _ptr(out)), "qg_pack_bits")
    return out


def unpack_bits(bits: int, buf: np.ndarray, count: int) -> np.ndarray:
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    if buf.size < (count * bits + 7) // 8:
        raise ValueError("buffer too short")
    out = np.empty(count, np.uint8)
    _check(_lib.qg_unpack_bits(bits, _ptr(buf), count, _ptr(out)), "qg_unpack_bits")
    return out


def quantize(fmt, w: np.ndarray) -> np.ndarray:
    """fp32 W [n, k] -> canonical encoding (uint8, qg_canonical_bytes bytes)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    out = np.empty(canonical_bytes(fmt, n, k), np.uint8)
    _check(_lib.qg_quantize(_fmt(fmt), _ptr(w), n, k, k, _ptr(out)), "qg_quantize")
    return out


def to_device_layout(fmt, canonical: np.ndarray, n: int, k: int) -> np.ndarray:
    canonical = np.ascontiguousarray(canonical, dtype=np.uint8)
    if canonical.size != canonical_bytes(fmt, n, k):
        raise ValueError("canonical buffer has the wrong size")
    out = np.empty(device_layout(fmt, n, k).total_bytes, np.uint8)
    _check(_lib.qg_to_device_layout(_fmt(fmt), _ptr(canonical), n, k, _ptr(out)), "qg_to_device_layout")
    return out


def from_device_layout(fmt, dev: np.ndarray, n: int, k: int) -> np.ndarray:
    dev = np.ascontiguousarray(dev, dtype=np.uint8)
    if dev.size != device_layout(fmt, n, k).total_bytes:
        raise ValueError("device-layout buffer has the wrong size")
    out = np.empty(canonical_bytes(fmt, n, k), np.uint8)
    _check(_lib.qg_from_device_layout(_fmt(fmt), _ptr(dev), n, k, _ptr(out)), "qg_from_device_layout")
    return out


# ---------------------------------------------------------------- device -------------------

def _torch():
    import torch
    return torch


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def upload(fmt, w: np.ndarray, device="cuda") -> "torch.Tensor":
    """Quantize fp32 W on the host, lay it out for the device and copy it to `device`."""
    torch = _torch()
    n, k = w.shape
    dev = to_device_layout(fmt, quantize(fmt, w), n, k)
    return torch.from_numpy(dev).to(device)


def to_device(fmt, canonical: np.ndarray, n: int, k: int, device="cuda") -> "torch.Tensor":
    torch = _torch()
    return torch.from_numpy(to_device_layout(fmt, canonical, n, k)).to(device)


def gemv(fmt, w, x, n: int, k: int, out=None, out_f32: bool = False, stream=None):
    """y = W_hat x. w: uint8 device buffer (device layout), x: fp16 [k] -> y fp16/fp32 [n]."""
    torch = _torch()
    if out is None:
        out = torch.empty(n, dtype=torch.float32 if out_f32 else torch.float16, device=x.device)
    _check(_lib.qg_gemv(_fmt(fmt), w.data_ptr(), x.data_ptr(), out.data_ptr(), int(out.dtype == torch.float32),
                        n, k, _stream(stream)), "qg_gemv")
    return out


def gemv_batched(fmt, w, w_stride: int, x, y, count: int, n: int, k: int, stream=None):
    """count independent GEMVs: W_b at w + b*w_stride bytes, x_b = x[b], y_b = y[b]."""
    torch = _torch()
    _check(_lib.qg_gemv_batched(_fmt(fmt), w.data_ptr(), w_stride, x.data_ptr(), x.stride(0), y.data_ptr(),
                                y.stride(0), int(y.dtype == torch.float32), count, n, k, _stream(stream)),
           "qg_gemv_batched")
    return y


def gemm(fmt, w, X, n: int, k: int, out=None, out_f32: bool = False, stream=None):
    """Y = X W_hat^T. w: uint8 device buffer (device layout), X: fp16 [m, k] (row stride
    X.stride(0)) -> Y fp16/fp32 [m, n]."""
    torch = _torch()
    m = X.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32 if out_f32 else torch.float16, device=X.device)
    _check(_lib.qg_gemm(_fmt(fmt), w.data_ptr(), X.data_ptr(), X.stride(0), out.data_ptr(), out.stride(0),
                        int(out.dtype == torch.float32), m, n, k, _stream(stream)), "qg_gemm")
    return out


def gemm_act_order(fmt, w, X, perm, n: int, k: int, out=None, out_f32: bool = False, stream=None):
    """Y = X[:, perm] W_hat^T for weights quantized with their columns permuted (stored column c
    is original column perm[c]). X: fp16 [m, k] (m <= 8) or [k]; perm: int32 [k] on the device."""
    torch = _torch()
    vec = X.dim() == 1
    m = 1 if vec else X.shape[0]
    if out is None:
        out = torch.empty((n,) if vec else (m, n), dtype=torch.float32 if out_f32 else torch.float16, device=X.device)
    if perm.dtype != torch.int32:
        raise TypeError("perm must be int32")
    _check(_lib.qg_gemm_act_order(_fmt(fmt), w.data_ptr(), X.data_ptr(), k if vec else X.stride(0), perm.data_ptr(),
                                  out.data_ptr(), n if vec else out.stride(0), int(out.dtype == torch.float32), m, n, k,
                                  _stream(stream)), "qg_gemm_act_order")
    return out


def gemm_grouped(fmt, ws, Xs, shapes, outs=None, out_f32: bool = False, stream=None):
    """One launch over several matrices: outs[g] = Xs[g] W_hat_g^T for W_g of shapes[g] = (n, k)
    at ws[g] (device layout). Every Xs[g] is fp16 [m, k_g] (one m, at most 8, row stride
    X.stride(0)) or [k_g] for m = 1; outs[g] is [m, n_g] (or [n_g]), allocated when None."""
    torch = _torch()
    count = len(ws)
    if not (len(Xs) == len(shapes) == count):
        raise ValueError("ws, Xs and shapes must have one entry per matrix")
    vec = Xs[0].dim() == 1
    m = 1 if vec else Xs[0].shape[0]
    dt = torch.float32 if out_f32 else torch.float16
    if outs is None:
        outs = [torch.empty((n,) if vec else (m, n), dtype=dt, device=X.device) for X, (n, _) in zip(Xs, shapes)]
    arr = lambda ctype, vals: (ctype * max(count, 1))(*vals)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    _check(_lib.qg_gemm_grouped(
        _fmt(fmt), count, arr(vp, [w.data_ptr() for w in ws]), arr(vp, [X.data_ptr() for X in Xs]),
        arr(i64, [X.stride(0) if X.dim() == 2 else X.shape[0] for X in Xs]), arr(vp, [y.data_ptr() for y in outs]),
        arr(i64, [y.stride(0) if y.dim() == 2 else y.shape[0] for y in outs]), arr(i64, [n for n, _ in shapes]),
        arr(i64, [k for _, k in shapes]), m, int(outs[0].dtype == torch.float32), _stream(stream)), "qg_gemm_grouped")
    return outs


def kv_quantize(x, codes=None, scales=None, stream=None):
    """8-bit KV-cache groups: fp16 [rows, cols] (row stride x.stride(0), cols % 32 == 0) ->
    (int8 codes [rows, cols], fp16 scales [rows, cols / 32])."""
    torch = _torch()
    rows, cols = x.shape
    if codes is None:
        codes = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // 32), dtype=torch.float16, device=x.device)
    _check(_lib.qg_kv_quantize(x.data_ptr(), x.stride(0), rows, cols, codes.data_ptr(), scales.data_ptr(),
                               _stream(stream)), "qg_kv_quantize")
    return codes, scales


def kv_dequantize(codes, scales, out=None, stream=None):
    """int8 codes [rows, cols] and fp16 scales [rows, cols / 32] -> fp16 [rows, cols]."""
    torch = _torch()
    rows, cols = codes.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float16, device=codes.device)
    _check(_lib.qg_kv_dequantize(codes.data_ptr(), scales.data_ptr(), rows, cols, out.data_ptr(), out.stride(0),
                                 _stream(stream)), "qg_kv_dequantize")
    return out


def dequantize(fmt, w, n: int, k: int, values: bool = True, codes: bool = True, stream=None):
    """Decode the device layout on the device: (W_hat fp32 [n, k] or None, codes uint8 [n, k] or None)."""
    torch = _torch()
    wv = torch.empty((n, k), dtype=torch.float32, device=w.device) if values else None
    cv = torch.empty((n, k), dtype=torch.uint8, device=w.device) if codes else None
    _check(_lib.qg_dequantize(_fmt(fmt), w.data_ptr(), wv.data_ptr() if values else None,
                              cv.data_ptr() if codes else None, n, k, _stream(stream)), "qg_dequantize")
    return wv, cv


def read_probe(buf, nbytes: int, sink, stream=None) -> None:
    """Stream nbytes of a device buffer through non-temporal 128-bit loads (read-ceiling measurement)."""
    _check(_lib.qg_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), _stream(stream)), "qg_read_probe")
