"""Helpers for the GPU parity tests: move synthetic layers to the device, run
the library, and compare with the oracle under the acceptance rule

    |y_gpu - y_ref| <= 2e-3 * sum_k |x_k W_kn| + 1e-3 * |y_ref|   (every element)
"""
from __future__ import annotations

import sys

import numpy as np

import oracle

REL_A = 2e-3
REL_Y = 1e-3


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
        "x": torch.from_numpy(L.x).to(dev),
        "bias": torch.from_numpy(L.bias).to(dev) if L.bias is not None else None,
    }
    return t


def make_matrix(L, t=None, g_idx="layer"):
    import gptq_bit_weight_amd as q4
    t = t or device_tensors(L)
    gi = t["g_idx"] if g_idx == "layer" else g_idx
    return q4.Q4Matrix(t["qweight"], t["qzeros"], t["scales"], gi, groupsize=L.G if L.G != L.K else -1)


def run(L, *, path=0, variant=0, splits=0, W=None, t=None, x=None, bias="layer"):
    torch = torch_mod()
    t = t or device_tensors(L)
    W = W or make_matrix(L, t)
    xb = t["x"] if x is None else x
    b = t["bias"] if bias == "layer" else bias
    y = W.matmul(xb, b, path=path, variant=variant, splits=splits)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def compare(y16: np.ndarray, y_ref: np.ndarray, A: np.ndarray, what: str = "") -> None:
    y = y16.astype(np.float64)
    err = np.abs(y - y_ref)
    tol = REL_A * A + REL_Y * np.abs(y_ref)
    bad = ~(err <= tol)
    if bad.any():
        idx = np.argwhere(bad)
        i = tuple(idx[0])
        ratio = float(np.max(np.where(tol > 0, err / np.maximum(tol, 1e-300), np.inf)))
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} elements outside tolerance; first at {i}: "
            f"gpu={y[i]!r} ref={y_ref[i]!r} A={A[i]!r}; worst err/tol={ratio:.3g}")


def oracle_full(L):
    return oracle.matmul(L.x, L.qweight, L.qzeros, L.scales, L.g_idx, L.K, L.N, L.G, bias=L.bias)


def oracle_sampled(L, ms, ns):
    return oracle.matmul_at(L.x, L.qweight, L.qzeros, L.scales, L.g_idx, L.K, L.N, L.G, ms, ns,
                            bias=L.bias)


def sample_indices(M: int, N: int, count: int, seed: int):
    """Sampled output elements: corners, the last row/column, random ones."""
    rng = np.random.default_rng(seed)
    ms = [0, M - 1, 0, M - 1]
    ns = [0, 0, N - 1, N - 1]
    ms += list(rng.integers(0, M, count))
    ns += list(rng.integers(0, N, count))
    return np.array(ms, dtype=np.int64), np.array(ns, dtype=np.int64)
