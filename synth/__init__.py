"""Seeded synthetic inputs for the GPTQ 4-bit linear layer.

This module is shared by the tests, the benchmark and the smoke check. It
serves both the CPU oracle and the HIP library, so it holds none of the
method's arithmetic: no unpacking, no dequantization, no products. It only
draws random tensors of the right dtype, shape and value distribution.

Tensor formats (the GPTQ checkpoint layout, "GPTQ's 'Exllama Kernel Not
Installed' Warning", section "Why the kernel is missing": 32-bit words
carrying 4-bit codes, with a scale and a zero point for every group; the I/O
contract table of "Implementation: Predibase Lorax GPTQ Exllama V1"):

- ``qweight`` int32 ``[K/8, N]``: word (r, n) holds the 4-bit codes of rows
  k = 8r .. 8r+7 of column n, code of k = 8r+i in bits 4i .. 4i+3.
- ``qzeros``  int32 ``[ceil(K/G), N/8]``: word (g, c) holds the zero points of
  columns n = 8c .. 8c+7 of group g, in the same nibble order.
- ``scales``  fp16  ``[ceil(K/G), N]``.
- ``g_idx``   int32 ``[K]`` or ``None`` (group of input row k).
- ``x``       fp16  ``[M, K]``, ``bias`` fp16 ``[N]``; or, with
  ``xfmt="bf16"``, both as bfloat16 bit patterns (uint16), the same draws
  rounded to bfloat16 instead (scales stay fp16).

Uniform 4-bit codes are drawn as uniform 32-bit words: the eight nibbles of
a uniformly random 32-bit word are independent and uniform on {0..15}, which
is exactly "q ~ U{0..15}, then packed" without any packing code here. With
``bits=8`` the words hold four 8-bit codes (qweight ``[K/4, N]``, qzeros
``[ceil(K/G), N/4]``), again uniform.

Draw order per layer (fixed so that a seed names one tensor set): qweight
words, qzeros words, scales, x, bias (if asked), act-order permutation (if
asked). Scales ~ U[0.005, 0.02] rounded to fp16, x ~ N(0, 1) rounded to
fp16, bias ~ N(0, 0.1) rounded to fp16. Act-order: a seeded permutation pi
of 0..K-1 and g_idx[k] = (position of k in pi) // G, so every group keeps
exactly G members but they are scattered over K.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Optional

import numpy as np

__all__ = [
    "Layer",
    "layer_seed",
    "make_layer",
    "make_x",
    "to_bf16_bits",
    "LLAMA7B_BLOCK",
    "LLAMA70B_MLP",
    "WORKLOADS",
]


@dataclasses.dataclass
class Layer:
    """One synthetic quantized linear layer plus an activation batch."""

    K: int
    N: int
    G: int
    qweight: np.ndarray           # int32 [K/8, N]
    qzeros: np.ndarray            # int32 [ceil(K/G), N/8]
    scales: np.ndarray            # float16 [ceil(K/G), N]
    g_idx: Optional[np.ndarray]   # int32 [K] or None
    x: np.ndarray                 # float16 [M, K] (xfmt "bf16": uint16 bfloat16 bits)
    bias: Optional[np.ndarray]    # float16 [N] or None (xfmt "bf16": uint16 bits)
    seed: int
    xfmt: str = "f16"
    bits: int = 4                 # 4 or 8 (qweight [K*bits/32, N], qzeros [ng, N*bits/32])

    @property
    def M(self) -> int:
        return int(self.x.shape[0])

    @property
    def n_groups(self) -> int:
        return -(-self.K // self.G)

    def metric_bytes(self) -> int:
        """Bytes of packed weights + scales + packed zeros (the streamed state)."""
        return int(self.qweight.nbytes + self.scales.nbytes + self.qzeros.nbytes)


def layer_seed(*parts) -> int:
    """Stable 32-bit seed from a tuple of names/numbers (crc32, not hash())."""
    return zlib.crc32("/".join(str(p) for p in parts).encode()) & 0xFFFFFFFF


def _words(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.integers(0, 1 << 32, size=shape, dtype=np.uint64).astype(np.uint32).view(np.int32)


def to_bf16_bits(values) -> np.ndarray:
    """Random draws as bfloat16 bit patterns (uint16): the float32 value's
    upper half, rounded to nearest with ties to even (finite inputs; input
    preparation only)."""
    u = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def make_layer(K: int, N: int, G: int, M: int, seed: int, *, act_order: bool = False,
               bias: bool = False, scale_lo: float = 0.005, scale_hi: float = 0.02,
               xfmt: str = "f16", bits: int = 4) -> Layer:
    """Draw one layer with the value distributions described in the module doc."""
    if xfmt not in ("f16", "bf16"):
        raise ValueError(f"unknown activation format {xfmt!r}")
    if bits not in (4, 8):
        raise ValueError(f"bits must be 4 or 8, got {bits}")
    if K % 8 or N % 8:
        raise ValueError("K and N must be multiples of 8")
    if G <= 0:
        G = K
    ng = -(-K // G)
    rng = np.random.Generator(np.random.PCG64(seed))
    per = 32 // bits
    qweight = _words(rng, (K // per, N))
    qzeros = _words(rng, (ng, N // per))
    scales = rng.uniform(scale_lo, scale_hi, size=(ng, N)).astype(np.float16)
    if xfmt == "f16":
        x = rng.standard_normal((M, K)).astype(np.float16)
        b = rng.normal(0.0, 0.1, size=(N,)).astype(np.float16) if bias else None
    else:
        x = to_bf16_bits(rng.standard_normal((M, K)))
        b = to_bf16_bits(rng.normal(0.0, 0.1, size=(N,))) if bias else None
    g_idx = None
    if act_order:
        pi = rng.permutation(K)
        pos = np.empty(K, dtype=np.int64)
        pos[pi] = np.arange(K)
        g_idx = (pos // G).astype(np.int32)
    return Layer(K=K, N=N, G=G, qweight=qweight, qzeros=qzeros, scales=scales,
                 g_idx=g_idx, x=x, bias=b, seed=seed, xfmt=xfmt, bits=bits)


def concat_layers(parts, x: Optional[np.ndarray] = None) -> Layer:
    """The layers `parts` (same K, G and g_idx) side by side: their packed
    weights, packed zeros, scales and biases concatenated along N, in part
    order, with one shared activation batch (parts[0].x unless given). A part
    without bias contributes zeros. Pure data plumbing, as QKV or gate/up
    projections that take the same input are stacked."""
    p0 = parts[0]
    for p in parts[1:]:
        if p.K != p0.K or p.G != p0.G:
            raise ValueError("parts must share K and G")
        if p.xfmt != p0.xfmt or p.bits != p0.bits:
            raise ValueError("parts must share the activation format and bit width")
        if (p.g_idx is None) != (p0.g_idx is None) or (
                p.g_idx is not None and not np.array_equal(p.g_idx, p0.g_idx)):
            raise ValueError("parts must share g_idx")
    bias = None
    if any(p.bias is not None for p in parts):
        zero = np.float16 if p0.xfmt == "f16" else np.uint16       # +0 either way
        bias = np.concatenate([p.bias if p.bias is not None else np.zeros(p.N, zero)
                               for p in parts])
    return Layer(K=p0.K, N=sum(p.N for p in parts), G=p0.G,
                 qweight=np.ascontiguousarray(np.concatenate([p.qweight for p in parts], axis=1)),
                 qzeros=np.ascontiguousarray(np.concatenate([p.qzeros for p in parts], axis=1)),
                 scales=np.ascontiguousarray(np.concatenate([p.scales for p in parts], axis=1)),
                 g_idx=p0.g_idx, x=p0.x if x is None else x, bias=bias, seed=p0.seed,
                 xfmt=p0.xfmt, bits=p0.bits)


def make_x(M: int, K: int, seed: int) -> np.ndarray:
    """A fresh fp16 activation batch x ~ N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((M, K)).astype(np.float16)


# Llama-7B-shaped decoder block: q, k, v, o (4096x4096), gate, up (4096x11008),
# down (11008x4096); bias on the q projection only. LLAMA7B_FUSED groups the
# layers that take the same input (q/k/v, gate/up) for one call each.
LLAMA7B_BLOCK = [
    ("q_proj", 4096, 4096, True),
    ("k_proj", 4096, 4096, False),
    ("v_proj", 4096, 4096, False),
    ("o_proj", 4096, 4096, False),
    ("gate_proj", 4096, 11008, False),
    ("up_proj", 4096, 11008, False),
    ("down_proj", 11008, 4096, False),
]
LLAMA7B_FUSED = [("qkv_proj", ("q_proj", "k_proj", "v_proj")), ("o_proj", ("o_proj",)),
                 ("gate_up_proj", ("gate_proj", "up_proj")), ("down_proj", ("down_proj",))]

# Llama-70B-shaped MLP layers (gate/up share a shape).
LLAMA70B_MLP = [
    ("gate_proj", 8192, 28672),
    ("down_proj", 28672, 8192),
]

# The five workloads, by name.
WORKLOADS = {
    "tiny": dict(K=512, N=512, G=128, M=[1]),
    "llama7b_block_decode": dict(layers=LLAMA7B_BLOCK, G=128, M=[1]),
    "llama7b_actorder": dict(shapes=[(4096, 11008), (11008, 4096)], G=128, M=[1, 4]),
    "llama70b_mlp_decode": dict(layers=LLAMA70B_MLP, G=128, M=[1, 2, 4, 8, 16]),
    "prefill": dict(shapes=[(4096, 11008), (11008, 4096)], G=[128, 32], M=[2048]),
}
