"""Test-side packer for 4-bit and 8-bit codes (pure Python/numpy, written
independently of the oracle and of the GPU library).

It builds GPTQ words from known codes so that tests can start from the codes
themselves rather than from an unpacking routine. Layout: qweight word (r, n)
holds the code of row k = 8r+i in bits 4i..4i+3; qzeros word (g, c) holds the
zero of column n = 8c+j in bits 4j..4j+3 (the packing stated for the tiny-layer
workload; "GPTQ's 'Exllama Kernel Not Installed' Warning", section "Why the
kernel is missing", says only that 32-bit words carry the 4-bit codes).
"""
from __future__ import annotations

import numpy as np


def pack_rows(codes: np.ndarray, bits: int = 4) -> np.ndarray:
    """codes uint [K, N] (values below 2^bits) -> int32 [K*bits/32, N],
    packed along K: word r holds rows r*per .. r*per + per - 1, per = 32/bits,
    the first in the lowest bits."""
    per = 32 // bits
    codes = np.asarray(codes, dtype=np.uint32)
    K, N = codes.shape
    assert K % per == 0
    out = np.zeros((K // per, N), dtype=np.uint32)
    for i in range(per):
        out |= (codes[i::per, :] & np.uint32((1 << bits) - 1)) << np.uint32(bits * i)
    return out.view(np.int32)


def pack_cols(codes: np.ndarray, bits: int = 4) -> np.ndarray:
    """codes uint [R, N] (values below 2^bits) -> int32 [R, N*bits/32], packed
    along N in the same order."""
    per = 32 // bits
    codes = np.asarray(codes, dtype=np.uint32)
    R, N = codes.shape
    assert N % per == 0
    out = np.zeros((R, N // per), dtype=np.uint32)
    for j in range(per):
        out |= (codes[:, j::per] & np.uint32((1 << bits) - 1)) << np.uint32(bits * j)
    return out.view(np.int32)


def pack_word_py(nibbles) -> int:
    """Eight codes (first = lowest bits) -> the int32 value, by plain Python."""
    w = 0
    for i, v in enumerate(nibbles):
        w |= (int(v) & 0xF) << (4 * i)
    return w - (1 << 32) if w >= (1 << 31) else w
