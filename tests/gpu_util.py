"""Helpers for the GPU parity tests: move synthetic layers to the device, run
the library, and compare with the oracle under the acceptance rule

    |y_gpu - y_ref| <= 2e-3 * sum_k |x_k W_kn| + 1e-3 * |y_ref|   (every element)

for fp16 activations. With bfloat16 activations and outputs the output
rounding alone can reach 2^-8 |y| (8 significant bits against fp16's 11), so
the |y| term is 8e-3 (twice that, the margin the fp16 rule gives 2^-11); the
GEMM also rounds each weight once to bfloat16 (relative error <= 2^-8 per
product), so its A term is 2e-3 + 2^-8 ~= 6e-3. The skinny kernel keeps the
weights exact (scale applied in fp32) and takes the fp16 A term.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle

REL_A = 2e-3
REL_Y = 1e-3
BF16_REL_Y = 8e-3
BF16_GEMM_REL_A = 6e-3


def announce(msg: str) -> None:
    """Name the case on the real stderr before a GPU step (survives capture)."""
    print(f"[gpu-case] {msg}", file=sys.__stderr__, flush=True)


def torch_mod():
    import torch
    return torch


def device_tensors(L):
    torch = torch_mod()
    dev = torch.device("cuda", 0)
    t = {
        "qweight": torch.from_numpy(L.qweight).to(dev),
        "qzeros": torch.from_numpy(L.qzeros).to(dev),
        "scales": torch.from_numpy(L.scales).to(dev),
        "g_idx": torch.from_numpy(L.g_idx).to(dev) if L.g_idx is not None else None,
        "x": _act(torch, L.x, L.xfmt).to(dev),
        "bias": _act(torch, L.bias, L.xfmt).to(dev) if L.bias is not None else None,
    }
    return t


def _act(torch, a, xfmt):
    """numpy activations -> torch tensor of the layer's format (bfloat16 from
    its uint16 bit patterns)."""
    if xfmt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(a)


def to_float64(y, xfmt="f16") -> np.ndarray:
    """GPU output (torch tensor or numpy) -> float64 values."""
    if hasattr(y, "cpu"):
        torch = torch_mod()
        y = y.cpu()
        if y.dtype == torch.bfloat16:
            return oracle.bf16_to_double(y.view(torch.int16).numpy().view(np.uint16))
        y = y.numpy()
    if xfmt == "bf16":
        return oracle.bf16_to_double(y)
    return np.asarray(y).astype(np.float64)


def make_matrix(L, t=None, g_idx="layer"):
    import gptq_bit_weight_amd as q4
    t = t or device_tensors(L)
    gi = t["g_idx"] if g_idx == "layer" else g_idx
    return q4.Q4Matrix(t["qweight"], t["qzeros"], t["scales"], gi, groupsize=L.G if L.G != L.K else -1,
                       bits=L.bits)


def run(L, *, path=0, variant=0, splits=0, W=None, t=None, x=None, bias="layer"):
    torch = torch_mod()
    t = t or device_tensors(L)
    W = W or make_matrix(L, t)
    xb = t["x"] if x is None else x
    b = t["bias"] if bias == "layer" else bias
    y = W.matmul(xb, b, path=path, variant=variant, splits=splits)
    torch.cuda.synchronize()
    if L.xfmt == "bf16":
        return to_float64(y)
    return y.cpu().numpy()


def compare(y16: np.ndarray, y_ref: np.ndarray, A: np.ndarray, what: str = "",
            rel_a: float = REL_A, rel_y: float = REL_Y) -> None:
    y = y16.astype(np.float64)
    err = np.abs(y - y_ref)
    tol = rel_a * A + rel_y * np.abs(y_ref)
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)
        i = tuple(idx[0])
        ratio = float(np.max(np.where(tol > 0, err / np.maximum(tol, 1e-300), np.inf)))
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} elements outside tolerance; first at {i}: "
            f"gpu={y[i]!r} ref={y_ref[i]!r} A={A[i]!r}; worst err/tol={ratio:.3g}")


def oracle_full(L):
    return oracle.matmul(L.x, L.qweight, L.qzeros, L.scales, L.g_idx, L.K, L.N, L.G, bias=L.bias,
                         xfmt=L.xfmt, bits=L.bits)


def oracle_sampled(L, ms, ns):
    return oracle.matmul_at(L.x, L.qweight, L.qzeros, L.scales, L.g_idx, L.K, L.N, L.G, ms, ns,
                            bias=L.bias, xfmt=L.xfmt, bits=L.bits)


def tile_lines(extent: int, window: int, per_window: int, seed: int, first: bool = False) -> np.ndarray:
    """Indices along one output axis that hit every `window`-wide stretch:
    the last index of each stretch, `per_window` random ones inside it and,
    with `first`, its first index (sorted, without repeats)."""
    rng = np.random.default_rng(seed)
    out = []
    for lo in range(0, extent, window):
        hi = min(extent, lo + window)
        out.append(hi - 1)
        if first:
            out.append(lo)
        out += list(rng.integers(lo, hi, per_window))
    return np.unique(np.array(out, dtype=np.int64))


def check_rows_cols(L, y, what: str, seed: int = 0, **tol) -> int:
    """Every element of whole output rows and whole output columns against the
    oracle. Rows: the first, the last and one random row of each row tile of
    the GEMM (64 rows up to M = 512, else 256); columns: column 0 and, of each
    128-column tile, the last and one random column. The rows cover every
    column of their tiles and the columns every row, so each output tile and
    each stream-K split of it has whole checked rows and columns. Returns the
    number of elements compared."""
    y = np.asarray(y)
    rows = tile_lines(L.M, 64 if L.M <= 512 else 256, 1, seed + 1, first=True)
    cols = np.unique(np.concatenate([[0], tile_lines(L.N, 128, 1, seed + 2)]))
    rm, rn = np.meshgrid(rows, np.arange(L.N, dtype=np.int64), indexing="ij")
    cm, cn = np.meshgrid(np.arange(L.M, dtype=np.int64), cols, indexing="ij")
    ms = np.concatenate([rm.ravel(), cm.ravel()])
    ns = np.concatenate([rn.ravel(), cn.ravel()])
    yD, A = oracle_sampled(L, ms, ns)
    compare(y[ms, ns], yD, A, what, **tol)
    return int(ms.size)


def check_output(L, y, what: str, seed: int = 0, full_max_m: int = 32, **tol) -> int:
    """The acceptance rule on a whole GPU output: every element for
    M <= full_max_m (the oracle computes the whole product; 32 covers every M
    the skinny kernel serves), else whole rows and columns through
    check_rows_cols. Returns the number of elements compared."""
    y = np.asarray(y)
    if L.M <= full_max_m:
        yD, A = oracle_full(L)
        compare(y, yD, A, what, **tol)
        return int(y.size)
    return check_rows_cols(L, y, what, seed, **tol)


def sample_indices(M: int, N: int, count: int, seed: int):
    """Sampled output elements: corners, the last row/column, random ones."""
    rng = np.random.default_rng(seed)
    ms = [0, M - 1, 0, M - 1]
    ns = [0, 0, N - 1, N - 1]
    ms += list(rng.integers(0, M, count))
    ns += list(rng.integers(0, N, count))
    return np.array(ms, dtype=np.int64), np.array(ns, dtype=np.int64)
