"""Test-side packer for 4-bit codes (pure Python/numpy, written independently
of the oracle and of the GPU library).

It builds GPTQ words from known codes so that tests can start from the codes
themselves rather than from an unpacking routine. Layout: qweight word (r, n)
holds the code of row k = 8r+i in bits 4i..4i+3; qzeros word (g, c) holds the
zero of column n = 8c+j in bits 4j..4j+3 (the packing stated for the tiny-layer
workload; "GPTQ's 'Exllama Kernel Not Installed' Warning", section "Why the
kernel is missing", says only that codes are packed into 32-bit words).
"""
from __future__ import annotations

import numpy as np


def pack_rows(codes: np.ndarray) -> np.ndarray:
    """codes uint [K, N] (values 0..15) -> int32 [K/8, N], packed along K."""
    codes = np.asarray(codes, dtype=np.uint32)
    K, N = codes.shape
    assert K % 8 == 0
    out = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        out |= (codes[i::8, :] & 0xF) << np.uint32(4 * i)
    return out.view(np.int32)


def pack_cols(codes: np.ndarray) -> np.ndarray:
    """codes uint [R, N] (values 0..15) -> int32 [R, N/8], packed along N."""
    codes = np.asarray(codes, dtype=np.uint32)
    R, N = codes.shape
    assert N % 8 == 0
    out = np.zeros((R, N // 8), dtype=np.uint32)
    for j in range(8):
        out |= (codes[:, j::8] & 0xF) << np.uint32(4 * j)
    return out.view(np.int32)


def pack_word_py(nibbles) -> int:
    """Eight codes (first = lowest bits) -> the int32 value, by plain Python."""
    w = 0
    for i, v in enumerate(nibbles):
        w |= (int(v) & 0xF) << (4 * i)
    return w - (1 << 32) if w >= (1 << 31) else w
