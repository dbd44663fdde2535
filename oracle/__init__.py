"""CPU oracle for the fused GPTQ 4-bit dequantize-and-multiply (numpy front end).

TEST INFRASTRUCTURE. Only ``tests/``, the smoke check in ``__graft_entry__``
and the CPU-baseline leg of ``bench.py`` may import this package. The GPU
library does not, and the two share no code.

The arithmetic lives in ``q4_oracle.c`` (plain C, double accumulation); this
module only marshals numpy arrays. See the C file's header for the passages
each function follows and for the readings taken where the pages are silent.

Functions:
  half_to_double(bits)         exact binary16 -> float64
  double_to_half(values)       float64 -> binary16 bits, round to nearest even
  bf16_to_double(bits)         exact bfloat16 -> float64
  double_to_bf16(values)       float64 -> bfloat16 bits, round to nearest even
  unpack_qweight(qweight, K)   uint8 [K, N] codes
  unpack_qzeros(qzeros, N)     uint8 [ng, N] zero points
  (every function taking packed tensors has bits=4 (default) or 8)
  dequant32(...)               float32 [K, N], W = s * (q - z) (exact)
  dequant16(...)               uint16 [K, N], binary16 bits of RNE(W)
  dequant_bf16(...)            uint16 [K, N], bfloat16 bits of RNE(W)
  matmul(..., route, xfmt)     float64 y [M, N] (and A = sum |x*W|), fused or fallback;
                               x and bias as binary16 ("f16") or bfloat16 ("bf16") bits
  matmul_at(..., ms, ns, xfmt) float64 y, A at selected output elements
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(LIB_PATH)
    lib.q4o_half_to_double.argtypes = [ctypes.c_uint16]
    lib.q4o_half_to_double.restype = ctypes.c_double
    lib.q4o_double_to_half_rne.argtypes = [ctypes.c_double]
    lib.q4o_double_to_half_rne.restype = ctypes.c_uint16
    lib.q4o_half_to_double_array.argtypes = [_I, _P, _P]
    lib.q4o_double_to_half_array.argtypes = [_I, _P, _P]
    lib.q4o_num_groups.argtypes = [_I, _I]
    lib.q4o_num_groups.restype = ctypes.c_int
    _F = ctypes.c_int
    lib.q4o_unpack_qweight_ex.argtypes = [_P, _I, _I, _F, _P]
    lib.q4o_unpack_qzeros_ex.argtypes = [_P, _I, _I, _F, _P]
    lib.q4o_dequant32_ex.argtypes = [_P, _P, _P, _P, _I, _I, _I, _F, _P]
    lib.q4o_dequant16_ex.argtypes = [_P, _P, _P, _P, _I, _I, _I, _F, _P]
    lib.q4o_bf16_to_double_array.argtypes = [_I, _P, _P]
    lib.q4o_double_to_bf16_array.argtypes = [_I, _P, _P]
    lib.q4o_dequant_bf16_ex.argtypes = [_P, _P, _P, _P, _I, _I, _I, _F, _P]
    lib.q4o_matmul_fused_ex.argtypes = [_F, _F, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P]
    lib.q4o_matmul_fallback_ex.argtypes = [_F, _F, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P]
    lib.q4o_matmul_fused_at_ex.argtypes = [_F, _F, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                           _I, _P, _P, _P, _P]
    for f in ("q4o_unpack_qweight_ex", "q4o_unpack_qzeros_ex", "q4o_dequant32_ex",
              "q4o_dequant16_ex", "q4o_dequant_bf16_ex", "q4o_matmul_fused_ex",
              "q4o_matmul_fallback_ex", "q4o_matmul_fused_at_ex"):
        getattr(lib, f).restype = ctypes.c_int
    lib.q4o_num_threads.restype = ctypes.c_int
    lib.q4o_set_num_threads.argtypes = [ctypes.c_int]
    lib.q4o_set_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


class OracleError(ValueError):
    pass


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def _bits16(a):
    """fp16 array (or its uint16 bit view) -> contiguous uint16 bits."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    return np.ascontiguousarray(a, dtype=np.uint16)


def _check(rc: int, what: str):
    if rc == 1:
        raise OracleError(f"{what}: bad shape or argument")
    if rc == 2:
        raise OracleError(f"{what}: g_idx value out of range")
    if rc:
        raise OracleError(f"{what}: error {rc}")


def num_threads() -> int:
    return int(_load().q4o_num_threads())


def set_num_threads(n: int) -> int:
    """Threads for the oracle's parallel loops from now on; returns the
    previous count. Results do not depend on it."""
    if n < 1:
        raise OracleError(f"thread count must be >= 1, got {n}")
    return int(_load().q4o_set_num_threads(n))


def num_groups(K: int, G: int) -> int:
    return int(_load().q4o_num_groups(K, G))


def half_to_double(bits) -> np.ndarray:
    b = _bits16(bits)
    out = np.empty(b.shape, dtype=np.float64)
    _load().q4o_half_to_double_array(b.size, _ptr(b), _ptr(out))
    return out


def double_to_half(values) -> np.ndarray:
    """Round to binary16 (ties to even); returns uint16 bit patterns."""
    v = _c(values, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().q4o_double_to_half_array(v.size, _ptr(v), _ptr(out))
    return out


def bf16_to_double(bits) -> np.ndarray:
    b = _bits16(bits)
    out = np.empty(b.shape, dtype=np.float64)
    _load().q4o_bf16_to_double_array(b.size, _ptr(b), _ptr(out))
    return out


def double_to_bf16(values) -> np.ndarray:
    """Round to bfloat16 (ties to even); returns uint16 bit patterns."""
    v = _c(values, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().q4o_double_to_bf16_array(v.size, _ptr(v), _ptr(out))
    return out


_XFMT = {"f16": 0, "bf16": 1}


def _xfmt(xfmt: str) -> int:
    if xfmt not in _XFMT:
        raise OracleError(f"unknown activation format {xfmt!r}")
    return _XFMT[xfmt]


def unpack_qweight(qweight, K: int, bits: int = 4) -> np.ndarray:
    qw = _c(qweight, np.int32)
    N = qw.shape[1]
    q = np.empty((K, N), dtype=np.uint8)
    _check(_load().q4o_unpack_qweight_ex(_ptr(qw), K, N, bits, _ptr(q)), "unpack_qweight")
    return q


def unpack_qzeros(qzeros, N: int, bits: int = 4) -> np.ndarray:
    qz = _c(qzeros, np.int32)
    ng = qz.shape[0]
    z = np.empty((ng, N), dtype=np.uint8)
    _check(_load().q4o_unpack_qzeros_ex(_ptr(qz), ng, N, bits, _ptr(z)), "unpack_qzeros")
    return z


def _weights(qweight, qzeros, scales, g_idx):
    return _c(qweight, np.int32), _c(qzeros, np.int32), _bits16(scales), _c(g_idx, np.int32)


def dequant32(qweight, qzeros, scales, g_idx, K: int, N: int, G: int, bits: int = 4) -> np.ndarray:
    qw, qz, s, gi = _weights(qweight, qzeros, scales, g_idx)
    W = np.empty((K, N), dtype=np.float32)
    _check(_load().q4o_dequant32_ex(_ptr(qw), _ptr(qz), _ptr(s), _ptr(gi), K, N, G, bits, _ptr(W)),
           "dequant32")
    return W


def dequant16(qweight, qzeros, scales, g_idx, K: int, N: int, G: int, bits: int = 4) -> np.ndarray:
    """binary16 bit patterns (uint16) of RNE(s * (q - z))."""
    qw, qz, s, gi = _weights(qweight, qzeros, scales, g_idx)
    dq = np.empty((K, N), dtype=np.uint16)
    _check(_load().q4o_dequant16_ex(_ptr(qw), _ptr(qz), _ptr(s), _ptr(gi), K, N, G, bits,
                                    _ptr(dq)), "dequant16")
    return dq


def dequant_bf16(qweight, qzeros, scales, g_idx, K: int, N: int, G: int, bits: int = 4) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of RNE(s * (q - z))."""
    qw, qz, s, gi = _weights(qweight, qzeros, scales, g_idx)
    dq = np.empty((K, N), dtype=np.uint16)
    _check(_load().q4o_dequant_bf16_ex(_ptr(qw), _ptr(qz), _ptr(s), _ptr(gi), K, N, G, bits,
                                       _ptr(dq)), "dequant_bf16")
    return dq


def matmul(x, qweight, qzeros, scales, g_idx, K: int, N: int, G: int, bias=None,
           route: str = "fused", xfmt: str = "f16", bits: int = 4
           ) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """y = x @ W (+ bias) in float64. Returns (y, A) for the fused route, where
    A[m, n] = sum_k |x[m,k] * W[k,n]|, and (y, None) for the fallback route.
    x and bias are bit patterns in format xfmt ("f16" or "bf16")."""
    fmt = _xfmt(xfmt)
    xb = _bits16(x)
    M = xb.shape[0]
    if xb.shape != (M, K):
        raise OracleError("x must be [M, K]")
    qw, qz, s, gi = _weights(qweight, qzeros, scales, g_idx)
    b = _bits16(bias)
    y = np.empty((M, N), dtype=np.float64)
    lib = _load()
    if route == "fused":
        A = np.empty((M, N), dtype=np.float64)
        _check(lib.q4o_matmul_fused_ex(fmt, bits, _ptr(xb), _ptr(qw), _ptr(qz), _ptr(s), _ptr(gi),
                                       _ptr(b), M, K, N, G, _ptr(y), _ptr(A)), "matmul_fused")
        return y, A
    if route == "fallback":
        _check(lib.q4o_matmul_fallback_ex(fmt, bits, _ptr(xb), _ptr(qw), _ptr(qz), _ptr(s),
                                          _ptr(gi), _ptr(b), M, K, N, G, _ptr(y)), "matmul_fallback")
        return y, None
    raise OracleError(f"unknown route {route!r}")


def matmul_at(x, qweight, qzeros, scales, g_idx, K: int, N: int, G: int, ms, ns,
              bias=None, xfmt: str = "f16", bits: int = 4) -> Tuple[np.ndarray, np.ndarray]:
    """Fused-route y and A at output elements (ms[i], ns[i])."""
    fmt = _xfmt(xfmt)
    xb = _bits16(x)
    M = xb.shape[0]
    qw, qz, s, gi = _weights(qweight, qzeros, scales, g_idx)
    b = _bits16(bias)
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    y = np.empty(ms.shape, dtype=np.float64)
    A = np.empty(ms.shape, dtype=np.float64)
    _check(_load().q4o_matmul_fused_at_ex(fmt, bits, _ptr(xb), _ptr(qw), _ptr(qz), _ptr(s),
                                          _ptr(gi), _ptr(b), M, K, N, G, ms.size, _ptr(ms),
                                          _ptr(ns), _ptr(y), _ptr(A)),
           "matmul_fused_at")
    return y, A


def within_tolerance(y_gpu, y_ref, A, rel_a: float = 2e-3, rel_y: float = 1e-3) -> np.ndarray:
    """Element-wise acceptance |y_gpu - y_ref| <= rel_a * A + rel_y * |y_ref|."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    return np.abs(y_gpu - y_ref) <= rel_a * A + rel_y * np.abs(y_ref)
