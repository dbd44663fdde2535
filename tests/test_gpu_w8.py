"""8-bit weights on the GPU (GPTQModel wiki "Inference Backends": GPTQ
kernels declare 4- and 8-bit weights; the native 8-bit path keeps the same
checkpoint tensors). Four codes a word, packed as the 4-bit codes; the
private layout stores a k-step's eight codes in two words.

 - the dequantized values of both kernels (fp16 and bfloat16 forms) bit-exact
   with the oracle's;
 - a layer whose 8-bit codes are all below 16 gives bit for bit the 4-bit
   layer's output with the same launch (same accumulation order, the same
   exact q - z or RNE(s (q - z)) operands);
 - parity with the oracle on both kernels, fp16 and bfloat16 activations,
   act-order (staged and permuted), symmetric layers, fused handles and a
   7B-shaped layer at full size (every element at M <= 2, whole rows and
   columns at M = 2048); argument errors.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (BF16_GEMM_REL_A, BF16_REL_Y, REL_A, REL_Y, announce, check_output,
                            compare, device_tensors, make_matrix, oracle_full, run, torch_mod)
from tests.packing import pack_cols, pack_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_bit_weight_amd as q4
    q4.load_library()
    yield


def _layer(K, N, G, M, seed, **kw):
    kw.setdefault("scale_lo", 0.0005)          # 8-bit codes: |q - z| up to 255
    kw.setdefault("scale_hi", 0.002)
    return synth.make_layer(K, N, G, M, seed=synth.layer_seed("w8", K, N, G, M, seed), bits=8, **kw)


def _tol(L, path):
    import gptq_bit_weight_amd as q4
    if L.xfmt == "bf16":
        return dict(rel_a=REL_A if path == q4.PATH_GEMV else BF16_GEMM_REL_A, rel_y=BF16_REL_Y)
    return dict(rel_a=REL_A, rel_y=REL_Y)


@pytest.mark.parametrize("K,N,G,act,sym", [(512, 512, 128, False, False), (1024, 264, 32, True, False),
                                           (160, 72, -1, False, False), (960, 136, 64, False, True)])
def test_w8_dequant_dump_bit_exact(K, N, G, act, sym):
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    L = _layer(K, N, G, 1, 0, act_order=act)
    announce(f"w8 dump K={K} N={N} G={G} act={act} sym={sym}")
    t = device_tensors(L)
    if sym:
        t["qzeros"] = None
    W = make_matrix(L, t)
    assert W.bits == 8
    qz = None if sym else L.qzeros
    ref16 = oracle.dequant16(L.qweight, qz, L.scales, L.g_idx, L.K, L.N, L.G, bits=8)
    refb = oracle.dequant_bf16(L.qweight, qz, L.scales, L.g_idx, L.K, L.N, L.G, bits=8)
    for path in (q4.PATH_GEMV, q4.PATH_MFMA):
        got = W.dequant_dump(path).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ref16), f"fp16 path {path}: {np.sum(got != ref16)} differ"
        got = W.dequant_dump(path, dtype=torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, refb), f"bf16 path {path}: {np.sum(got != refb)} differ"


@pytest.mark.parametrize("M,path", [(1, 1), (5, 1), (16, 1), (40, 2), (300, 2)])
def test_w8_small_codes_equal_4bit_layer(M, path):
    """Codes and zeros below 16: the 8-bit handle and the 4-bit handle of the
    same codes give the same output bit for bit (one column tile, no split,
    the GEMM on both)."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    rng = np.random.default_rng(M)
    K, N, G = 1024, 200, 128
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    z = rng.integers(0, 16, size=(K // G, N), dtype=np.uint8)
    L = synth.make_layer(K, N, G, M, seed=M, bias=True)
    announce(f"w8 vs w4 M={M} path={path}")
    dev = torch.device("cuda", 0)
    sc = torch.from_numpy(L.scales).to(dev)
    W4 = q4.Q4Matrix(torch.from_numpy(pack_rows(q)).to(dev), torch.from_numpy(pack_cols(z)).to(dev), sc,
                     None, G)
    W8 = q4.Q4Matrix(torch.from_numpy(pack_rows(q, 8)).to(dev), torch.from_numpy(pack_cols(z, 8)).to(dev),
                     sc, None, G, bits=8)
    x = torch.from_numpy(L.x).to(dev)
    b = torch.from_numpy(L.bias).to(dev)
    kw = dict(path=path, variant=1, splits=1) if path == 1 else dict(path=path, variant=3)
    y4, y8 = W4.matmul(x, b, **kw), W8.matmul(x, b, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y4.view(torch.int16), y8.view(torch.int16))


GEMV_CASES = [
    # K, N, G, M, act_order, bias, xfmt
    (512, 512, 128, 1, False, False, "f16"),
    (1024, 1096, 128, 1, False, True, "f16"),     # ragged column tiles
    (1024, 1096, 32, 3, False, False, "f16"),     # groups of 32
    (2048, 200, 64, 16, False, True, "f16"),      # M at the skinny limit
    (96, 8, 32, 2, False, False, "f16"),          # K tail inside a block
    (160, 72, -1, 5, False, False, "f16"),        # one group over K
    (1024, 264, 128, 1, True, True, "f16"),       # act-order, staged in the kernel
    (1024, 264, 128, 4, True, True, "f16"),       # act-order, separate permute
    (1024, 1096, 128, 2, False, True, "bf16"),
    (1024, 264, 32, 9, True, False, "bf16"),
    (1024, 1096, 128, 20, False, True, "f16"),    # two row blocks
    (1024, 264, 64, 31, True, False, "bf16"),     # two row blocks, act-order
]


@pytest.mark.parametrize("tiles", [0, 1, 2])
@pytest.mark.parametrize("K,N,G,M,act,bias,xfmt", GEMV_CASES)
def test_w8_gemv_parity(K, N, G, M, act, bias, xfmt, tiles):
    import gptq_bit_weight_amd as q4
    L = _layer(K, N, G, M, 1, act_order=act, bias=bias, xfmt=xfmt)
    announce(f"w8 gemv K={K} N={N} G={G} M={M} act={act} {xfmt} tiles={tiles}")
    y = run(L, path=q4.PATH_GEMV, variant=tiles)
    yD, A = oracle_full(L)
    compare(y, yD, A, f"w8 gemv K={K} N={N} M={M}", **_tol(L, q4.PATH_GEMV))


@pytest.mark.parametrize("splits", [2, 5])
def test_w8_gemv_splits(splits):
    import gptq_bit_weight_amd as q4
    L = _layer(4096, 64, 128, 3, 2, bias=True)
    announce(f"w8 splits={splits}")
    y = run(L, path=q4.PATH_GEMV, splits=splits)
    yD, A = oracle_full(L)
    compare(y, yD, A, f"w8 splits={splits}", **_tol(L, q4.PATH_GEMV))


GEMM_CASES = [
    (512, 328, 128, 17, False, False, "f16"),
    (512, 328, 32, 130, False, True, "f16"),
    (96, 136, 32, 300, False, False, "f16"),      # K tail inside the 64-row k-tile
    (1024, 256, 128, 256, True, True, "f16"),     # act-order
    (320, 72, -1, 33, False, False, "f16"),
    (512, 328, 128, 70, False, True, "bf16"),
    (1024, 256, 32, 256, True, False, "bf16"),
]


@pytest.mark.parametrize("K,N,G,M,act,bias,xfmt", GEMM_CASES)
def test_w8_gemm_parity(K, N, G, M, act, bias, xfmt):
    import gptq_bit_weight_amd as q4
    L = _layer(K, N, G, M, 3, act_order=act, bias=bias, xfmt=xfmt)
    announce(f"w8 gemm K={K} N={N} G={G} M={M} act={act} {xfmt}")
    y = run(L, path=q4.PATH_MFMA)
    yD, A = oracle_full(L)
    compare(y, yD, A, f"w8 gemm K={K} N={N} M={M}", **_tol(L, q4.PATH_MFMA))


def test_w8_symmetric_and_fused():
    """Symmetric parts (zero point 128) in a fused handle: each column equals
    its own part's handle, and the whole matches the oracle."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    parts = [_layer(2048, n, 128, 4, 10 + i, bias=True) for i, n in enumerate((256, 136))]
    cat = synth.concat_layers(parts)
    announce("w8 fused symmetric")
    dev = [device_tensors(p) for p in parts]
    W = q4.Q4Matrix.concat([(d["qweight"], None, d["scales"]) for d in dev], groupsize=128, bits=8)
    tc = device_tensors(cat)
    y = W.matmul(tc["x"], tc["bias"], path=q4.PATH_GEMV, variant=1, splits=1)
    singles = [q4.Q4Matrix(d["qweight"], None, d["scales"], None, 128, bits=8)
               .matmul(tc["x"], d["bias"], path=q4.PATH_GEMV, variant=1, splits=1) for d in dev]
    torch.cuda.synchronize()
    for got, ref in zip(W.split(y), singles):
        assert torch.equal(got.contiguous().view(torch.int16), ref.view(torch.int16))
    yD, A = oracle.matmul(cat.x, cat.qweight, None, cat.scales, None, cat.K, cat.N, 128, bias=cat.bias,
                          bits=8)
    compare(y.cpu().numpy(), yD, A, "w8 fused symmetric")


@pytest.mark.parametrize("K,N,M", [(4096, 11008, 1), (11008, 4096, 2), (4096, 11008, 2048)])
def test_w8_full_size(K, N, M):
    import gptq_bit_weight_amd as q4
    L = _layer(K, N, 128, M, 4, bias=True)
    announce(f"w8 full K={K} N={N} M={M}")
    W = make_matrix(L)
    path = W.path_for(M)
    y = run(L, W=W)
    W.close()
    check_output(L, y, f"w8 full {K}x{N} M={M}", seed=M, **_tol(L, path))


def test_w8_argument_errors():
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    L = _layer(256, 64, 128, 20, 5)
    announce("w8 errors")
    t = device_tensors(L)
    W = make_matrix(L, t)
    with pytest.raises(NotImplementedError, match="2 column tiles"):
        W.matmul(t["x"][:4].contiguous(), path=q4.PATH_GEMV, variant=4)
    with pytest.raises(ValueError, match="not 0, 3, 4 or 8"):
        W.matmul(t["x"], path=q4.PATH_MFMA, variant=2)
    with pytest.raises(NotImplementedError):
        q4.Q4Matrix(t["qweight"], t["qzeros"], t["scales"], None, 128, bits=6)
    with pytest.raises(ValueError):        # 4-bit shapes for an 8-bit handle
        q4.Q4Matrix(t["qweight"], t["qzeros"][:, :4].contiguous(), t["scales"], None, 128, bits=8)
