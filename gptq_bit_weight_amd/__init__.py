"""Python binding of libq4: the fused GPTQ 4-bit dequantize-and-multiply on
AMD Instinct MI355X (gfx950).

The binding only marshals arguments: it checks dtype, device, shape and
contiguity of torch tensors, passes their device pointers and the current
HIP stream to the C ABI (``include/q4.h``) and turns status codes into
exceptions. Every step of the computation runs in the library's HIP kernels;
there is no Python or CPU fallback -- if ``libq4.so`` is missing or fails to
load, importing the library raises.

    import gptq_bit_weight_amd as q4
    W = q4.Q4Matrix(qweight, qzeros, scales, g_idx, groupsize=128)   # q4_make
    y = W.matmul(x)                                                   # q4_matmul
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "Q4Matrix", "Q4Error", "load_library", "library_path", "check_shape", "plan_actorder",
    "plan_gemv", "plan_gemv_gather", "plan_gemm", "PATH_NONE", "PATH_GEMV", "PATH_MFMA", "GEMV_MAX_M", "EXPORTED_SYMBOLS",
]

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "libq4.so")

PATH_NONE, PATH_GEMV, PATH_MFMA = 0, 1, 2
GEMV_MAX_M = 32          # Q4_GEMV_MAX_M: most rows the skinny kernel takes
GEMM_MAX_WORKERS = 1024
STATIC_SCRATCH_BYTES = 64 << 20     # Q4_STATIC_SCRATCH_BYTES: q4_matmul_static's per-GPU array

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_DEVICE, ERR_HIP, ERR_OOM = range(6)

# Every function include/q4.h declares.
EXPORTED_SYMBOLS = (
    "q4_make", "q4_make_cat", "q4_matmul", "q4_matmul_bias", "q4_matmul_ex", "q4_free", "q4_last_status",
    "q4_last_error", "q4_path_for", "q4_dequant_dump", "q4_handle_info", "q4_check_shape",
    "q4_plan_actorder", "q4_plan_gemv", "q4_gemv_gather", "q4_plan_gemv_gather",
    "q4_matmul_bf16", "q4_matmul_ex_bf16", "q4_dequant_dump_bf16", "q4_make_bits", "q4_make_cat_bits",
    "q4_handle_bits", "q4_check_shape_bits", "q4_plan_gemm", "q4_plan_gemm_waves", "q4_read_probe",
    "q4_matmul_static",
)

_lib = None


class Q4Error(RuntimeError):
    """A libq4 call failed with Q4_ERR_HIP or Q4_ERR_OOM."""


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libq4.so (once). Raises ImportError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run: python -m gptq_bit_weight_amd.build")
    try:
        lib = ctypes.CDLL(_LIB_PATH)
    except OSError as e:
        raise ImportError(f"cannot load {_LIB_PATH}: {e}") from e
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.q4_make.argtypes = [P, P, P, P, I, I, I]
    lib.q4_make.restype = P
    lib.q4_make_cat.argtypes = [I, P, P, P, P, I, P, I]
    lib.q4_make_cat.restype = P
    lib.q4_make_bits.argtypes = [P, P, P, P, I, I, I, I]
    lib.q4_make_bits.restype = P
    lib.q4_make_cat_bits.argtypes = [I, P, P, P, P, I, P, I, I]
    lib.q4_make_cat_bits.restype = P
    lib.q4_handle_bits.argtypes = [P]
    lib.q4_handle_bits.restype = I
    lib.q4_check_shape_bits.argtypes = [I, I, I, I]
    lib.q4_check_shape_bits.restype = I
    lib.q4_matmul.argtypes = [P, P, P, I, P]
    lib.q4_matmul_bias.argtypes = [P, P, P, P, I, P]
    lib.q4_matmul_ex.argtypes = [P, P, P, P, I, I, I, I, P]
    lib.q4_matmul_bf16.argtypes = [P, P, P, P, I, P]
    lib.q4_matmul_static.argtypes = [P, P, P, P, I, P]
    lib.q4_matmul_ex_bf16.argtypes = [P, P, P, P, I, I, I, I, P]
    for f in (lib.q4_matmul, lib.q4_matmul_bias, lib.q4_matmul_ex, lib.q4_matmul_bf16,
              lib.q4_matmul_ex_bf16, lib.q4_matmul_static):
        f.restype = I
    lib.q4_free.argtypes = [P]
    lib.q4_free.restype = None
    lib.q4_last_status.argtypes = []
    lib.q4_last_status.restype = I
    lib.q4_last_error.argtypes = []
    lib.q4_last_error.restype = ctypes.c_char_p
    lib.q4_path_for.argtypes = [P, I]
    lib.q4_path_for.restype = I
    lib.q4_dequant_dump.argtypes = [P, I, P, P]
    lib.q4_dequant_dump.restype = I
    lib.q4_dequant_dump_bf16.argtypes = [P, I, P, P]
    lib.q4_dequant_dump_bf16.restype = I
    lib.q4_handle_info.argtypes = [P, ctypes.POINTER(I), ctypes.POINTER(I), ctypes.POINTER(I),
                                   ctypes.POINTER(I)]
    lib.q4_handle_info.restype = I
    lib.q4_check_shape.argtypes = [I, I, I]
    lib.q4_check_shape.restype = I
    lib.q4_plan_actorder.argtypes = [P, I, I, P, ctypes.POINTER(I)]
    lib.q4_plan_actorder.restype = I
    lib.q4_plan_gemv.argtypes = [I, I, I, I, I, ctypes.POINTER(I), ctypes.POINTER(I)]
    lib.q4_plan_gemv.restype = I
    lib.q4_gemv_gather.argtypes = [P, I, I]
    lib.q4_gemv_gather.restype = I
    lib.q4_plan_gemv_gather.argtypes = [I, I, I]
    lib.q4_plan_gemv_gather.restype = I
    lib.q4_plan_gemm.argtypes = [I, I, I, I]
    lib.q4_plan_gemm.restype = I
    lib.q4_plan_gemm_waves.argtypes = [I, I, I, I]
    lib.q4_plan_gemm_waves.restype = I
    lib.q4_read_probe.argtypes = [P, ctypes.c_size_t, P, P]
    lib.q4_read_probe.restype = I
    _lib = lib
    return lib


def _raise(status: int, what: str):
    msg = (load_library().q4_last_error() or b"").decode(errors="replace")
    text = f"{what}: {msg}" if msg else what
    if status == ERR_INVALID_ARG:
        raise ValueError(text)
    if status in (ERR_UNSUPPORTED, ERR_DEVICE):
        raise NotImplementedError(text)
    raise Q4Error(text)


def _check(status: int, what: str):
    if status != OK:
        _raise(status, what)


# ---------------------------------------------------------------- host only ---

def check_shape(K: int, N: int, groupsize: int, bits: int = 4) -> None:
    """Raise if (K, N, groupsize) is not accepted by q4_make (q4_make_bits)."""
    if bits == 4:
        _check(load_library().q4_check_shape(K, N, groupsize), "q4_check_shape")
    else:
        _check(load_library().q4_check_shape_bits(K, N, groupsize, bits), "q4_check_shape_bits")


def plan_actorder(g_idx, K: int, groupsize: int):
    """Host act-order plan: returns (perm, trivial) for an int32 g_idx (numpy)."""
    import numpy as np
    g = np.ascontiguousarray(g_idx, dtype=np.int32)
    if g.shape != (K,):
        raise ValueError("g_idx must have shape [K]")
    perm = np.empty(K, dtype=np.int32)
    triv = ctypes.c_int(0)
    _check(load_library().q4_plan_actorder(g.ctypes.data, K, groupsize, perm.ctypes.data,
                                           ctypes.byref(triv)), "q4_plan_actorder")
    return perm, bool(triv.value)


def plan_gemv(M: int, K: int, N: int, groupsize: int, num_cu: int = 256) -> tuple:
    """(column tiles per wave, K splits) the skinny kernel uses for this shape
    on a chip of num_cu CUs."""
    lib = load_library()
    ct, sp = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib.q4_plan_gemv(M, K, N, groupsize, num_cu, ctypes.byref(ct), ctypes.byref(sp)),
           "q4_plan_gemv")
    return int(ct.value), int(sp.value)


def plan_gemm(M: int, N: int, K: int, num_cu: int = 256) -> int:
    """Workgroups of the streaming GEMM for an M x N output with K rows, at
    the planned tile width: the number of output tiles (one each; 64 x 128
    when M <= 512, else 256 x 128 or 256 x 256) or a stream-K count
    (q4_plan_gemm)."""
    r = int(load_library().q4_plan_gemm(M, N, K, num_cu))
    if r < 0:
        raise ValueError(f"q4_plan_gemm: bad arguments M={M} N={N} K={K}")
    return r


def plan_gemm_waves(M: int, N: int, K: int, num_cu: int = 256) -> int:
    """The streaming GEMM's planned tile width in waves of 32 columns: 8
    (256-column tiles) or 4 (128-column tiles) (q4_plan_gemm_waves)."""
    r = int(load_library().q4_plan_gemm_waves(M, N, K, num_cu))
    if r < 0:
        raise ValueError(f"q4_plan_gemm_waves: bad arguments M={M} N={N} K={K}")
    return r


def plan_gemv_gather(M: int, K: int, splits: int) -> bool:
    """Whether the skinny kernel builds act-order activations x[:, perm] in
    LDS itself for this M, K and number of K splits (only unsplit launches
    with M <= 2 whose activations fit 40 KiB)."""
    r = int(load_library().q4_plan_gemv_gather(M, K, splits))
    if r < 0:
        raise ValueError(f"q4_plan_gemv_gather: bad arguments M={M} K={K} splits={splits}")
    return bool(r)


# ---------------------------------------------------------------- device ---

def _torch():
    import torch
    return torch


def _dev_tensor(t, dtype, name: str, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _stream_ptr(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


class Q4Matrix:
    """A 4-bit GPTQ weight matrix prepared for the MI355X kernels (q4_make).

    qweight int32 [K/8, N], qzeros int32 [K/G, N/8] (None for a symmetric
    layer stored without zeros: every zero point is 8), scales fp16 [K/G, N],
    g_idx int32 [K] or None; all on the current GPU, contiguous. The handle
    keeps its own copy in a private layout; later edits of the tensors do
    not reach it.
    """

    def __init__(self, qweight, qzeros, scales, g_idx=None, groupsize: int = 128, bits: int = 4):
        self._build([(qweight, qzeros, scales)], g_idx, groupsize, bits)

    @classmethod
    def concat(cls, parts, g_idx=None, groupsize: int = 128, bits: int = 4):
        """One matrix over the column concatenation of layers that share the
        input (QKV or gate/up fusion; q4_make_cat). parts: sequence of
        (qweight, qzeros, scales) with equal K; g_idx shared by all parts.
        Output columns follow part order; split() cuts an output into parts."""
        self = cls.__new__(cls)
        self._build(list(parts), g_idx, groupsize, bits)
        return self

    def _build(self, parts, g_idx, groupsize, bits=4):
        torch = _torch()
        lib = load_library()
        if not parts:
            raise ValueError("at least one part is needed")
        if bits not in (4, 8):
            raise NotImplementedError(f"bits must be 4 or 8, got {bits}")
        per = 32 // bits                # codes per int32 word
        K = None
        ns = []
        for i, (qweight, qzeros, scales) in enumerate(parts):
            _dev_tensor(qweight, torch.int32, f"qweight[{i}]")
            if qweight.dim() != 2:
                raise ValueError(f"qweight must be 2-D [K/{per}, N]")
            k_i, n_i = int(qweight.shape[0]) * per, int(qweight.shape[1])
            if K is not None and k_i != K:
                raise ValueError(f"part {i} has K={k_i}, part 0 has K={K}")
            K = k_i
            check_shape(K, n_i, groupsize, bits)
            G = K if groupsize == -1 else groupsize
            ng = -(-K // G) if G > 0 else 0
            if qzeros is not None:      # None: symmetric, every zero point is 2^(bits-1)
                _dev_tensor(qzeros, torch.int32, f"qzeros[{i}]", (ng, n_i // per))
            _dev_tensor(scales, torch.float16, f"scales[{i}]", (ng, n_i))
            ns.append(n_i)
        check_shape(K, sum(ns), groupsize, bits)
        if g_idx is not None:
            _dev_tensor(g_idx, torch.int32, "g_idx", (K,))
        dev = parts[0][0].device
        for i, part in enumerate(parts):
            for t, nm in zip(part, ("qweight", "qzeros", "scales")):
                if t is not None and t.device != dev:
                    raise ValueError(f"{nm}[{i}] is on {t.device}, qweight[0] on {dev}")
        if g_idx is not None and g_idx.device != dev:
            raise ValueError(f"g_idx is on {g_idx.device}, qweight[0] on {dev}")
        gp = g_idx.data_ptr() if g_idx is not None else None
        with torch.cuda.device(dev):
            if len(parts) == 1:
                qw, qz, sc = parts[0]
                h = lib.q4_make_bits(qw.data_ptr(), qz.data_ptr() if qz is not None else None,
                                     sc.data_ptr(), gp, K, ns[0], groupsize, bits)
                what = "q4_make_bits"
            else:
                arr = lambda vals: (ctypes.c_void_p * len(vals))(*vals)
                h = lib.q4_make_cat_bits(len(parts), arr([p[0].data_ptr() for p in parts]),
                                         arr([p[1].data_ptr() if p[1] is not None else None for p in parts]),
                                         arr([p[2].data_ptr() for p in parts]), gp, K,
                                         (ctypes.c_int * len(ns))(*ns), groupsize, bits)
                what = "q4_make_cat_bits"
        if not h:
            _raise(lib.q4_last_status(), what)
        self._h = ctypes.c_void_p(h)
        self.K, self.N, self.device = K, sum(ns), dev
        self.part_n = tuple(ns)
        gs, act = ctypes.c_int(0), ctypes.c_int(0)
        lib.q4_handle_info(self._h, None, None, ctypes.byref(gs), ctypes.byref(act))
        self.groupsize = int(gs.value)
        self.act_order = bool(act.value)
        self.bits = int(lib.q4_handle_bits(self._h))

    def split(self, out):
        """Views of an output [M, N] as one [M, N_i] per part (column order)."""
        views, off = [], 0
        for n in self.part_n:
            views.append(out[:, off:off + n])
            off += n
        return views

    def _handle(self):
        if self._h is None:
            raise ValueError("Q4Matrix is closed")
        return self._h

    def path_for(self, M: int) -> int:
        return int(load_library().q4_path_for(self._handle(), M))

    def gemv_gather(self, M: int, splits: int = 0) -> bool:
        """For an act-order handle: whether the skinny kernel builds x[:, perm]
        in LDS itself at this M and K splits (0: planned), rather than a
        separate permute kernel running first."""
        r = int(load_library().q4_gemv_gather(self._handle(), M, splits))
        if r < 0:
            raise ValueError(f"q4_gemv_gather: bad arguments M={M} splits={splits}")
        return bool(r)

    def matmul(self, x, bias=None, out=None, *, path: int = 0, variant: int = 0, splits: int = 0,
               stream=None):
        """out[M, N] = x[M, K] @ W (+ bias), accumulated in fp32 and rounded
        once to the activations' dtype: float16, or bfloat16 (bias and out
        then bfloat16 too; the weights and fp16 scales are the same).

        path: 0 automatic, PATH_GEMV or PATH_MFMA. variant: skinny kernel --
        16-column tiles per wave (0 planned, 1, 2, 4); GEMM -- the tile
        width: 0 or 3 planned (plan_gemm_waves), 4 (128 columns) or 8 (256
        columns, M > 512 only).
        splits: skinny kernel K splits (0 planned, 1..16); GEMM workgroups
        (0 planned, 1 one per output tile, 2..GEMM_MAX_WORKERS sharing the
        tiles' k-steps: stream-K)."""
        torch = _torch()
        h = self._handle()
        if getattr(x, "dtype", None) not in (torch.float16, torch.bfloat16):
            raise ValueError(f"x must be float16 or bfloat16, got {getattr(x, 'dtype', type(x))}")
        dt = x.dtype
        _dev_tensor(x, dt, "x")
        if x.dim() != 2 or x.shape[1] != self.K:
            raise ValueError(f"x must be [M, {self.K}], got {tuple(x.shape)}")
        M = int(x.shape[0])
        if out is None:
            out = torch.empty((M, self.N), dtype=dt, device=x.device)
        else:
            _dev_tensor(out, dt, "out", (M, self.N))
        if bias is not None:
            _dev_tensor(bias, dt, "bias", (self.N,))
        for t, nm in ((x, "x"), (out, "out"), (bias, "bias")):
            if t is not None and t.device != self.device:
                raise ValueError(f"{nm} is on {t.device}, the matrix on {self.device}")
        lib = load_library()
        fn, name = ((lib.q4_matmul_ex_bf16, "q4_matmul_bf16") if dt == torch.bfloat16
                    else (lib.q4_matmul_ex, "q4_matmul"))
        with torch.cuda.device(self.device):
            st = fn(h, x.data_ptr(), bias.data_ptr() if bias is not None else None,
                    out.data_ptr(), M, path, variant, splits, _stream_ptr(stream))
        _check(st, name)
        return out

    __call__ = matmul

    def matmul_static(self, x, bias=None, out=None, *, stream=None):
        """q4_matmul_static: as matmul(x, bias, out) for float16 activations
        with the automatic launch, allocating no device memory (every
        workspace is the library's static per-GPU array; calls that overlap
        on one GPU race). `out` must be given by callers that cannot let
        torch allocate."""
        torch = _torch()
        h = self._handle()
        _dev_tensor(x, torch.float16, "x")
        if x.dim() != 2 or x.shape[1] != self.K:
            raise ValueError(f"x must be [M, {self.K}], got {tuple(x.shape)}")
        M = int(x.shape[0])
        if out is None:
            out = torch.empty((M, self.N), dtype=torch.float16, device=x.device)
        else:
            _dev_tensor(out, torch.float16, "out", (M, self.N))
        if bias is not None:
            _dev_tensor(bias, torch.float16, "bias", (self.N,))
        for t, nm in ((x, "x"), (out, "out"), (bias, "bias")):
            if t is not None and t.device != self.device:
                raise ValueError(f"{nm} is on {t.device}, the matrix on {self.device}")
        with torch.cuda.device(self.device):
            st = load_library().q4_matmul_static(h, x.data_ptr(), bias.data_ptr() if bias is not None else None,
                                                 out.data_ptr(), M, _stream_ptr(stream))
        _check(st, "q4_matmul_static")
        return out

    def dequant_dump(self, path: int = PATH_GEMV, stream=None, dtype=None):
        """[K, N] in dtype (float16, or bfloat16 for the bfloat16 kernels): the
        dequantized values the kernel of `path` computes."""
        torch = _torch()
        dtype = dtype or torch.float16
        if dtype not in (torch.float16, torch.bfloat16):
            raise TypeError(f"dtype must be float16 or bfloat16, got {dtype}")
        w = torch.empty((self.K, self.N), dtype=dtype, device=self.device)
        lib = load_library()
        fn = lib.q4_dequant_dump_bf16 if dtype == torch.bfloat16 else lib.q4_dequant_dump
        with torch.cuda.device(self.device):
            st = fn(self._handle(), path, w.data_ptr(), _stream_ptr(stream))
        _check(st, "q4_dequant_dump")
        return w

    def close(self):
        if getattr(self, "_h", None) is not None:
            torch = _torch()
            torch.cuda.synchronize(self.device)
            load_library().q4_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
