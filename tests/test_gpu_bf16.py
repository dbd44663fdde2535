"""bfloat16 activations, bias and output on the GPU (GPTQModel wiki
"Inference Backends", hardware table, ExLlama v2 row: the activation dtype is
kept, scales stay FP16, accumulation is FP32).

 - the bfloat16 weights each kernel forms are bit-exact with the oracle's
   RNE_bf16(s * (q - z)) (debug dump, both kernels);
 - the skinny kernel and the GEMM against the oracle's bfloat16 route, every
   element, under the bfloat16 acceptance rule (tests/gpu_util.py): the
   skinny kernel keeps the exact weights (2e-3 A + 8e-3 |y|), the GEMM
   rounds them to bfloat16 (6e-3 A + 8e-3 |y|);
 - activations far beyond binary16's range;
 - act-order (in-kernel staging and the separate permute), fused handles,
   the 7B shapes at full size (every element at M = 1, whole rows and
   columns at M = 2048), argument errors.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (BF16_GEMM_REL_A, BF16_REL_Y, REL_A, announce, check_output, compare,
                            device_tensors, make_matrix, oracle_full, run, to_float64, torch_mod)

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
    return synth.make_layer(K, N, G, M, seed=synth.layer_seed("bf16", K, N, G, M, seed), xfmt="bf16",
                            **kw)


def _tol(path):
    import gptq_bit_weight_amd as q4
    return dict(rel_a=REL_A if path == q4.PATH_GEMV else BF16_GEMM_REL_A, rel_y=BF16_REL_Y)


@pytest.mark.parametrize("K,N,G,act,sym", [(512, 512, 128, False, False), (1024, 264, 32, True, False),
                                           (160, 72, -1, False, False), (960, 136, 64, False, True)])
def test_dequant_dump_bf16_bit_exact(K, N, G, act, sym):
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    L = _layer(K, N, G, 1, 0, act_order=act)
    announce(f"bf16 dump K={K} N={N} G={G} act={act} sym={sym}")
    t = device_tensors(L)
    if sym:
        t["qzeros"] = None
    W = make_matrix(L, t)
    qz = None if sym else L.qzeros
    ref = oracle.dequant_bf16(L.qweight, qz, L.scales, L.g_idx, L.K, L.N, L.G)
    for path in (q4.PATH_GEMV, q4.PATH_MFMA):
        got = W.dequant_dump(path, dtype=torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ref), f"path {path}: {np.sum(got != ref)} values differ"


GEMV_CASES = [
    # K, N, G, M, act_order, bias
    (512, 512, 128, 1, False, False),
    (1024, 1096, 128, 1, False, True),      # ragged column tiles, bias
    (1024, 1096, 32, 3, False, False),      # groups of 32
    (2048, 200, 64, 16, False, True),       # M at the skinny limit
    (96, 8, 32, 2, False, False),           # K tail inside a block, one column word
    (160, 72, -1, 5, False, False),         # one group over K
    (1024, 264, 128, 1, True, True),        # act-order staged in the kernel
    (1024, 264, 128, 4, True, True),        # act-order, separate permute
    (1024, 1096, 128, 30, False, True),     # two row blocks
    (1024, 264, 32, 32, True, False),       # two full row blocks, groups of 32, act-order
]


@pytest.mark.parametrize("tiles", [0, 2])
@pytest.mark.parametrize("K,N,G,M,act,bias", GEMV_CASES)
def test_gemv_bf16_parity(K, N, G, M, act, bias, tiles):
    import gptq_bit_weight_amd as q4
    L = _layer(K, N, G, M, 1, act_order=act, bias=bias)
    announce(f"bf16 gemv K={K} N={N} G={G} M={M} act={act} tiles={tiles}")
    y = run(L, path=q4.PATH_GEMV, variant=tiles)
    yD, A = oracle_full(L)
    compare(y, yD, A, f"bf16 gemv K={K} N={N} M={M}", **_tol(q4.PATH_GEMV))


GEMM_CASES = [
    (512, 328, 128, 17, False, False),
    (512, 328, 32, 130, False, True),
    (96, 136, 32, 300, False, False),       # K tail inside the 64-row k-tile
    (1024, 256, 128, 256, True, True),      # act-order
    (320, 72, -1, 33, False, False),
]


@pytest.mark.parametrize("K,N,G,M,act,bias", GEMM_CASES)
def test_gemm_bf16_parity(K, N, G, M, act, bias):
    import gptq_bit_weight_amd as q4
    L = _layer(K, N, G, M, 2, act_order=act, bias=bias)
    announce(f"bf16 gemm K={K} N={N} G={G} M={M} act={act}")
    y = run(L, path=q4.PATH_MFMA)
    yD, A = oracle_full(L)
    compare(y, yD, A, f"bf16 gemm K={K} N={N} M={M}", **_tol(q4.PATH_MFMA))


@pytest.mark.parametrize("M,path", [(2, 1), (40, 2)])
def test_bf16_beyond_binary16_range(M, path):
    """Activations around 1e6 (binary16 would overflow) and 1e-6 rows: the
    bfloat16 route keeps them."""
    torch = torch_mod()
    L = _layer(1024, 136, 128, M, 3, bias=True)
    xv = oracle.bf16_to_double(L.x)
    xv[0] *= 1e6
    xv[-1] *= 1e-6
    L.x = synth.to_bf16_bits(xv)
    announce(f"bf16 range M={M} path={path}")
    y = run(L, path=path)
    assert np.isfinite(y).all() and np.abs(y[0]).max() > 1e4
    yD, A = oracle_full(L)
    compare(y, yD, A, "bf16 range", **_tol(path))


def test_bf16_fused_handle():
    """A fused (concatenated) handle with bfloat16 activations: each column
    equals its own part's handle bit for bit."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    parts = [_layer(2048, n, 128, 4, 10 + i, bias=True) for i, n in enumerate((256, 128))]
    cat = synth.concat_layers(parts)
    announce("bf16 fused")
    dev = [device_tensors(p) for p in parts]
    W = q4.Q4Matrix.concat([(d["qweight"], d["qzeros"], d["scales"]) for d in dev], groupsize=128)
    tc = device_tensors(cat)
    y = W.matmul(tc["x"], tc["bias"], path=q4.PATH_GEMV, variant=1, splits=1)
    singles = [make_matrix(p, d).matmul(tc["x"], d["bias"], path=q4.PATH_GEMV, variant=1, splits=1)
               for p, d in zip(parts, dev)]
    torch.cuda.synchronize()
    for got, ref in zip(W.split(y), singles):
        assert torch.equal(got.contiguous().view(torch.int16), ref.view(torch.int16))
    yD, A = oracle_full(cat)
    compare(to_float64(y), yD, A, "bf16 fused", **_tol(q4.PATH_GEMV))


@pytest.mark.parametrize("K,N,M", [(4096, 11008, 1), (11008, 4096, 1), (4096, 11008, 2048)])
def test_bf16_llama7b_full_size(K, N, M):
    """The 7B MLP shapes at full size with the launch the automatic plan takes:
    every element at M = 1, whole rows and columns at M = 2048."""
    import gptq_bit_weight_amd as q4
    L = _layer(K, N, 128, M, 4, bias=True)
    announce(f"bf16 full K={K} N={N} M={M}")
    W = make_matrix(L)
    path = W.path_for(M)
    y = run(L, W=W)
    W.close()
    check_output(L, y, f"bf16 full {K}x{N} M={M}", seed=M, **_tol(path))


def test_bf16_argument_errors():
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    L = _layer(256, 64, 128, 20, 5, bias=True)
    announce("bf16 errors")
    t = device_tensors(L)
    W = make_matrix(L, t)
    with pytest.raises(ValueError, match="not 0, 3, 4 or 8"):
        W.matmul(t["x"], path=q4.PATH_MFMA, variant=1)
    with pytest.raises(ValueError):
        W.matmul(t["x"], t["bias"].to(torch.float16))      # bias must match x
    with pytest.raises(ValueError):
        W.matmul(t["x"], out=torch.empty((20, 64), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        W.matmul(t["x"].to(torch.float32))
    y = W.matmul(t["x"], t["bias"])
    assert y.dtype == torch.bfloat16
