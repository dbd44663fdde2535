"""GPU parity of libq4 against the CPU oracle (needs an MI355X).

Every test goes through the C ABI (via the ctypes binding) and compares with
the oracle on the same seeded inputs:
 - the dequantized fp16 values the kernels compute are bit-exact with the
   oracle's RNE(s * (q - z)) (debug dump);
 - every output element satisfies the acceptance rule in gpu_util;
 - invariants of the pages: trivial g_idx == no g_idx, act-order == the
   physically K-permuted layer ("Implementation: Predibase Lorax GPTQ
   Exllama V1", Description; GPTQModel wiki "Inference Backends", section
   "Runtime cache lifetime"), fused result == the dequantize-then-matmul
   fallback's answer ("GPTQ's 'Exllama Kernel Not Installed' Warning",
   section "What the fallback actually does": the oracle checks that one).
Sizes span several tiles of both kernels and ragged tails in M, N and K.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (announce, compare, device_tensors, make_matrix, oracle_full, run,
                            torch_mod)
from tests.packing import pack_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_bit_weight_amd as q4
    q4.load_library()            # must load where a GPU is present: no fallback
    yield


def _layer(K, N, G, M, seed, **kw):
    return synth.make_layer(K, N, G, M, seed=synth.layer_seed("parity", K, N, G, M, seed), **kw)


# ------------------------------------------------------------------ dequant --

@pytest.mark.parametrize("K,N,G,act", [(512, 512, 128, False), (1024, 264, 32, True),
                                       (768, 136, 64, False), (512, 72, 256, True),
                                       (96, 40, -1, False)])
def test_dequant_dump_bit_exact(K, N, G, act):
    import gptq_bit_weight_amd as q4
    L = _layer(K, N, G, 1, 0, act_order=act)
    announce(f"dump K={K} N={N} G={G} act={act}")
    W = make_matrix(L)
    assert W.act_order == act
    ref = oracle.dequant16(L.qweight, L.qzeros, L.scales, L.g_idx, L.K, L.N, L.G)
    for path in (q4.PATH_GEMV, q4.PATH_MFMA):
        got = W.dequant_dump(path).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ref), f"path {path}: {np.sum(got != ref)} values differ"


# ---------------------------------------------------------- skinny kernel --

GEMV_CASES = [
    # K, N, G, M, act_order, bias
    (512, 512, 128, 1, False, False),      # the tiny 512 x 512 layer
    (1024, 1096, 128, 1, False, True),     # 17.1 column tiles (ragged), bias
    (1024, 1096, 32, 3, False, False),     # groups of 32
    (2048, 200, 64, 16, False, True),      # M at the skinny limit
    (96, 8, 32, 2, False, False),          # K tail inside a 4-step batch, one column word
    (160, 72, -1, 5, False, False),        # one group over K (K not a multiple of 128)
    (1024, 264, 128, 4, True, True),       # act-order
    (768, 520, 256, 7, True, False),       # act-order, groups of 256
]


@pytest.mark.parametrize("tiles", [0, 1, 2, 4])
@pytest.mark.parametrize("K,N,G,M,act,bias", GEMV_CASES)
def test_gemv_parity(K, N, G, M, act, bias, tiles):
    """tiles: 16-column MFMA tiles per wave (0: planned)."""
    import gptq_bit_weight_amd as q4
    L = _layer(K, N, G, M, 1, act_order=act, bias=bias)
    announce(f"gemv K={K} N={N} G={G} M={M} act={act} bias={bias} tiles={tiles}")
    W = make_matrix(L)
    assert W.path_for(M) == q4.PATH_GEMV
    y = run(L, W=W, path=q4.PATH_GEMV, variant=tiles)
    yD, A = oracle_full(L)
    compare(y, yD, A, f"gemv K={K} N={N} G={G} M={M} tiles={tiles}")


# Past 16 rows the skinny kernel runs two blocks of 16 activation rows over
# each unpacked weight fragment.
GEMV_ROWS_CASES = [
    # K, N, G, M, act_order, bias
    (1024, 1096, 128, 17, False, True),    # the second row block one row
    (2048, 200, 64, 32, False, False),     # two full row blocks
    (1024, 264, 32, 25, False, True),      # groups of 32
    (160, 72, -1, 20, False, False),       # K tail, one group over K
    (1024, 264, 128, 32, True, True),      # act-order (separate permute)
    (768, 520, 256, 29, False, False),     # groups of 256
]


@pytest.mark.parametrize("tiles", [0, 1, 2, 4])
@pytest.mark.parametrize("K,N,G,M,act,bias", GEMV_ROWS_CASES)
def test_gemv_row_blocks_parity(K, N, G, M, act, bias, tiles):
    """The skinny kernel at 17 <= M <= 32 (tiles: 16-column MFMA tiles per
    wave, 0 planned)."""
    import gptq_bit_weight_amd as q4
    L = _layer(K, N, G, M, 7, act_order=act, bias=bias)
    announce(f"gemv rows K={K} N={N} G={G} M={M} act={act} bias={bias} tiles={tiles}")
    W = make_matrix(L)
    assert W.path_for(M) == q4.PATH_GEMV
    y = run(L, W=W, path=q4.PATH_GEMV, variant=tiles)
    yD, A = oracle_full(L)
    compare(y, yD, A, f"gemv rows K={K} N={N} G={G} M={M} tiles={tiles}")


@pytest.mark.parametrize("M", [17, 24, 32])
def test_row_blocks_splits_deterministic(M):
    """K splits with row blocks: the partial sums of every split and row
    reach the last arriver; repeated calls give the same bits."""
    import gptq_bit_weight_amd as q4
    L = _layer(2048, 136, 128, M, 8, bias=True)
    announce(f"row blocks splits M={M}")
    t = device_tensors(L)
    W = make_matrix(L, t)
    yD, A = oracle_full(L)
    for splits in (2, 3, 16):
        a = run(L, W=W, t=t, path=q4.PATH_GEMV, variant=1, splits=splits)
        b = run(L, W=W, t=t, path=q4.PATH_GEMV, variant=1, splits=splits)
        compare(a, yD, A, f"row blocks M={M} splits={splits}")
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_dispatch_by_m():
    """Automatic path: the skinny kernel up to 32 rows, the GEMM above; both
    agree with the oracle on either side of the boundary."""
    import gptq_bit_weight_amd as q4
    L = _layer(1024, 520, 128, 33, 9, bias=True)
    t = device_tensors(L)
    W = make_matrix(L, t)
    for M in (1, 16, 17, 32):
        assert W.path_for(M) == q4.PATH_GEMV, M
    for M in (33, 64, 65, 2048):
        assert W.path_for(M) == q4.PATH_MFMA, M
    yD, A = oracle_full(L)
    for M in (32, 33):
        announce(f"dispatch M={M}")
        y = W.matmul(t["x"][:M].contiguous(), t["bias"])
        torch_mod().cuda.synchronize()
        compare(y.cpu().numpy(), yD[:M], A[:M], f"dispatch M={M}")


# ------------------------------------------------------------ MFMA GEMM --

GEMM_CASES = [
    (512, 328, 128, 17, False, False),     # smallest M the GEMM takes, ragged N
    (512, 328, 32, 130, False, True),      # ragged M over two row tiles, groups of 32
    (96, 136, 32, 300, False, False),      # K tail inside the 64-row k-tile
    (1024, 256, 128, 256, True, True),     # act-order, whole tiles
    (768, 264, 256, 70, True, False),      # act-order, groups of 256
    (320, 72, -1, 33, False, False),       # one group over K
    (640, 200, 64, 90, False, True),       # groups of 64: one group per k-tile
]


@pytest.mark.parametrize("splits", [0, 1])
@pytest.mark.parametrize("K,N,G,M,act,bias", GEMM_CASES)
def test_gemm_parity(K, N, G, M, act, bias, splits):
    """splits 0: the planned launch (stream-K where planned); 1: one workgroup
    per output tile."""
    import gptq_bit_weight_amd as q4
    L = _layer(K, N, G, M, 2, act_order=act, bias=bias)
    announce(f"gemm K={K} N={N} G={G} M={M} act={act} bias={bias} splits={splits}")
    W = make_matrix(L)
    assert W.path_for(M) == (q4.PATH_GEMV if M <= 32 else q4.PATH_MFMA)
    y = run(L, W=W, path=q4.PATH_MFMA, splits=splits)
    yD, A = oracle_full(L)
    compare(y, yD, A, f"gemm K={K} N={N} G={G} M={M} splits={splits}")


def test_gemm_variant_names_one_kernel():
    """GEMM variant 0 (automatic) and 3 name the same kernel: bit-identical
    results."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    L = _layer(1024, 520, 128, 300, 21, bias=True)
    announce("gemm variants")
    t = device_tensors(L)
    W = make_matrix(L, t)
    a = W.matmul(t["x"], t["bias"], path=q4.PATH_MFMA, variant=0, splits=1)
    c = W.matmul(t["x"], t["bias"], path=q4.PATH_MFMA, variant=3, splits=1)
    torch.cuda.synchronize()
    assert torch.equal(a, c)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_both_kernels_agree_at_small_m(M):
    import gptq_bit_weight_amd as q4
    L = _layer(1024, 328, 128, M, 3, bias=True)
    announce(f"paths M={M}")
    t = device_tensors(L)
    W = make_matrix(L, t)
    yD, A = oracle_full(L)
    for path in (q4.PATH_GEMV, q4.PATH_MFMA):
        compare(run(L, W=W, t=t, path=path), yD, A, f"path {path} M={M}")


# ---------------------------------------------------------------- split-K --

@pytest.mark.parametrize("splits,tiles", [(1, 1), (2, 1), (3, 1), (4, 1), (5, 1), (8, 1),
                                          (16, 1), (3, 2), (4, 4), (16, 4)])
def test_splits_valid_and_deterministic(splits, tiles):
    L = _layer(2048, 200, 128, 3, 4, bias=True)
    announce(f"splits={splits} tiles={tiles}")
    t = device_tensors(L)
    W = make_matrix(L, t)
    yD, A = oracle_full(L)
    a = run(L, W=W, t=t, variant=tiles, splits=splits)
    b = run(L, W=W, t=t, variant=tiles, splits=splits)
    compare(a, yD, A, f"splits={splits} tiles={tiles}")
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_repeated_split_calls_reset_counters():
    """The split-K arrival counters are reset by the reducing workgroup, so
    many back-to-back calls keep giving the same answer."""
    torch = torch_mod()
    L = _layer(4096, 512, 128, 1, 5)
    announce("repeat splits")
    t = device_tensors(L)
    W = make_matrix(L, t)
    first = W.matmul(t["x"], splits=8)
    outs = [W.matmul(t["x"], splits=8) for _ in range(50)]
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), first.view(torch.int16))


# ------------------------------------------------------------- invariants --

def test_trivial_g_idx_bit_identical_to_none():
    torch = torch_mod()
    L = _layer(1024, 264, 128, 4, 6)
    announce("trivial g_idx")
    t = device_tensors(L)
    triv = torch.arange(1024, dtype=torch.int32, device="cuda") // 128
    W0 = make_matrix(L, t, g_idx=None)
    W1 = make_matrix(L, t, g_idx=triv)
    assert not W1.act_order
    for M, x in ((4, t["x"]), (40, torch.from_numpy(synth.make_x(40, 1024, 9)).cuda())):
        assert torch.equal(W0.matmul(x).view(torch.int16), W1.matmul(x).view(torch.int16))


@pytest.mark.parametrize("M", [1, 4, 64])
def test_act_order_bit_identical_to_physical_permutation(M):
    """A non-trivial g_idx gives exactly the output of a trivial layer built
    from the K-permuted weights and activations."""
    torch = torch_mod()
    L = _layer(1024, 200, 128, M, 7, act_order=True, bias=True)
    announce(f"act-order invariant M={M}")
    perm = np.argsort(L.g_idx, kind="stable")
    q = oracle.unpack_qweight(L.qweight, L.K)
    t = device_tensors(L)
    Wa = make_matrix(L, t)
    assert Wa.act_order
    Wp = make_matrix(L, dict(t, qweight=torch.from_numpy(pack_rows(q[perm])).cuda()), g_idx=None)
    xp = torch.from_numpy(np.ascontiguousarray(L.x[:, perm])).cuda()
    ya = Wa.matmul(t["x"], t["bias"])
    yp = Wp.matmul(xp, t["bias"])
    torch.cuda.synchronize()
    assert torch.equal(ya.view(torch.int16), yp.view(torch.int16))
    yD, A = oracle_full(L)
    compare(ya.cpu().numpy(), yD, A, "act-order")


@pytest.mark.parametrize("K,N,G,M,splits,tiles,gathers", [
    (1024, 200, 128, 1, 0, 0, True),   # staged in the kernel
    (1024, 200, 128, 2, 1, 2, True),   # two rows, two tiles
    (1024, 200, 64, 1, 0, 4, True),    # groups of 64, four tiles
    (992, 72, 32, 2, 1, 0, True),      # K not a multiple of 128: zero rows to the block end
    (1024, 200, 128, 1, 3, 0, False),  # split K: separate permute
    (1024, 200, 128, 3, 1, 0, False),  # M > 2: separate permute
    (12416, 64, 128, 1, 1, 0, False),  # 97 blocks exceed 12288 rows: separate permute
    (12288, 64, 128, 1, 1, 1, True),   # three 8-row units per thread
    (10112, 64, 128, 2, 1, 0, True),   # 2 x 10120 halfs: the LDS limit
])
def test_act_order_gather_matches_permuted_layer(K, N, G, M, splits, tiles, gathers):
    """The skinny kernel's own staging of x[:, perm] (or the separate permute,
    when it does not apply) gives the output of a trivial layer built from
    the K-permuted weights and activations with the same launch, bit for bit,
    and matches the oracle."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    L = _layer(K, N, G, M, 11, act_order=True, bias=True)
    announce(f"act-order staging K={K} N={N} G={G} M={M} splits={splits} tiles={tiles}")
    perm = np.argsort(L.g_idx, kind="stable")
    q = oracle.unpack_qweight(L.qweight, L.K)
    t = device_tensors(L)
    Wa = make_matrix(L, t)
    s = splits or q4.plan_gemv(M, K, N, G)[1]
    assert q4.plan_gemv_gather(M, K, s) == gathers and Wa.gemv_gather(M, splits) == gathers
    Wp = make_matrix(L, dict(t, qweight=torch.from_numpy(pack_rows(q[perm])).cuda()), g_idx=None)
    xp = torch.from_numpy(np.ascontiguousarray(L.x[:, perm])).cuda()
    ya = Wa.matmul(t["x"], t["bias"], path=q4.PATH_GEMV, variant=tiles, splits=splits)
    yp = Wp.matmul(xp, t["bias"], path=q4.PATH_GEMV, variant=tiles, splits=s)
    torch.cuda.synchronize()
    assert torch.equal(ya.view(torch.int16), yp.view(torch.int16))
    yD, A = oracle_full(L)
    compare(ya.cpu().numpy(), yD, A, "act-order staging")


def test_bias_is_added_once_in_fp32():
    torch = torch_mod()
    L = _layer(512, 136, 128, 2, 8, bias=True)
    announce("bias")
    t = device_tensors(L)
    W = make_matrix(L, t)
    y0 = W.matmul(t["x"]).float()
    yb = W.matmul(t["x"], t["bias"]).float()
    yD, A = oracle_full(L)
    compare(yb.cpu().numpy().astype(np.float16), yD, A, "bias")
    diff = (yb - y0 - t["bias"].float()).abs()
    assert float(diff.max()) <= float(2 ** -9 * (y0.abs().max() + 1))


# ------------------------------------------------------------ edge cases --

def test_m_zero_and_argument_errors():
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    L = _layer(256, 64, 128, 2, 10)
    announce("edges")
    t = device_tensors(L)
    W = make_matrix(L, t)
    assert W.path_for(0) == q4.PATH_NONE and W.path_for(16) == q4.PATH_GEMV
    assert W.path_for(32) == q4.PATH_GEMV and W.path_for(33) == q4.PATH_MFMA
    e = W.matmul(torch.empty((0, 256), dtype=torch.float16, device="cuda"))
    assert tuple(e.shape) == (0, 64)
    with pytest.raises(ValueError):
        W.matmul(t["x"].float())
    with pytest.raises(ValueError):
        W.matmul(torch.zeros((2, 128), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        W.matmul(torch.zeros((q4.GEMV_MAX_M + 1, 256), dtype=torch.float16, device="cuda"),
                 path=q4.PATH_GEMV)
    with pytest.raises(ValueError):
        W.matmul(t["x"], splits=17)
    with pytest.raises(ValueError):
        W.matmul(t["x"], path=q4.PATH_MFMA, splits=q4.GEMM_MAX_WORKERS + 1)
    for v in (1, 2, 5, 16):
        with pytest.raises(ValueError, match="not 0, 3, 4 or 8"):
            W.matmul(t["x"], path=q4.PATH_MFMA, variant=v)
    with pytest.raises(ValueError):
        W.matmul(t["x"], path=q4.PATH_GEMV, variant=3)
    bad = torch.full((256,), 3, dtype=torch.int32, device="cuda")      # only groups 0, 1
    with pytest.raises(ValueError, match="outside"):
        q4.Q4Matrix(t["qweight"], t["qzeros"], t["scales"], bad, groupsize=128)
    uneven = torch.arange(256, dtype=torch.int32, device="cuda") // 128
    uneven[0] = 1
    with pytest.raises(NotImplementedError, match="uniform"):
        q4.Q4Matrix(t["qweight"], t["qzeros"], t["scales"], uneven, groupsize=128)
    with pytest.raises(NotImplementedError):
        q4.Q4Matrix(t["qweight"], t["qzeros"], t["scales"], None, groupsize=100)
    # the handle is a snapshot: editing the source tensor afterwards changes nothing
    y1 = W.matmul(t["x"]).clone()
    t["qweight"].zero_()
    y2 = W.matmul(t["x"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_special_values_propagate():
    """Zero weights give exact zeros; an infinite scale gives inf/NaN only in
    its own column (IEEE propagation, no clamping)."""
    torch = torch_mod()
    K, N, G, M = 256, 64, 128, 3
    L = _layer(K, N, G, M, 11)
    z = oracle.unpack_qzeros(L.qzeros, N)
    # q == z everywhere in column 5 -> W[:, 5] == 0 -> y[:, 5] == 0 exactly
    q = oracle.unpack_qweight(L.qweight, K)
    q[:, 5] = np.repeat(z[:, 5], G)
    L.qweight = pack_rows(q)
    L.scales = L.scales.copy()
    L.scales[1, 9] = np.float16(np.inf)
    announce("special values")
    y = run(L)
    yD, A = oracle_full(L)
    assert np.all(y[:, 5] == 0)
    assert np.all(~np.isfinite(y[:, 9]))
    fin = np.isfinite(yD)
    keep = np.ones(N, dtype=bool)
    keep[9] = False
    compare(y[:, keep], yD[:, keep], A[:, keep], "special")
    assert fin[:, keep].all()


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("xfmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,path", [(1, 1), (2, 1), (16, 1), (24, 1), (40, 2)])
def test_zero_and_sparse_columns(M, path, xfmt, bits):
    """Degenerate columns against the acceptance rule, which scales with
    A = sum |x| |w| rather than with sum |x|: a column whose codes all equal
    their zero points (W = 0, so A = 0 and, without a bias, the output must
    be exactly 0), one with a single nonzero weight in the layer and one with
    a single nonzero weight in every 32-row k-step. A kernel whose rounding
    grew with sum |x| (for instance one that took the zero point out of the
    sum as (c + z) * sum x) fails these."""
    from tests.gpu_util import BF16_GEMM_REL_A, BF16_REL_Y, REL_A, REL_Y
    K, N, G = 1024, 128, 128
    L = _layer(K, N, G, M, 13, xfmt=xfmt, bits=bits)
    z = oracle.unpack_qzeros(L.qzeros, N, bits=bits)
    q = oracle.unpack_qweight(L.qweight, K, bits=bits)
    levels = 1 << bits
    for c in (3, 7, 11):
        q[:, c] = np.repeat(z[:, c], G)
    q[517, 7] = (int(z[517 // G, 7]) + 1) % levels
    for t in range(K // 32):
        k = 32 * t + (7 * t) % 32
        q[k, 11] = (int(z[k // G, 11]) + 3) % levels
    L.qweight = pack_rows(q, bits)
    announce(f"zero and sparse columns M={M} path={path} {xfmt} w{bits}")
    y = run(L, path=path)
    yD, A = oracle_full(L)
    assert A[:, 3].max() == 0 and np.all(y[:, 3] == 0)
    if xfmt == "bf16":
        tol = dict(rel_a=BF16_GEMM_REL_A if path == 2 else REL_A, rel_y=BF16_REL_Y)
    else:
        tol = dict(rel_a=REL_A, rel_y=REL_Y)
    compare(y, yD, A, f"zero/sparse columns M={M} {xfmt}", **tol)


# ------------------------------------------------------ format variants --

@pytest.mark.parametrize("M", [1, 6, 40])
def test_symmetric_layer_without_zeros(M):
    """qzeros absent: a symmetric layer whose zero points are all 8 (the
    oracle's reading of the "Missing zeros" row), on both kernels; the dump
    stays bit-exact and a fused handle may mix symmetric and stored-zero
    parts."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    L = _layer(1024, 200, 128, M, 31, bias=True)
    announce(f"symmetric M={M}")
    t = device_tensors(L)
    W = q4.Q4Matrix(t["qweight"], None, t["scales"], None, groupsize=128)
    y = W.matmul(t["x"], t["bias"])
    torch.cuda.synchronize()
    yD, A = oracle.matmul(L.x, L.qweight, None, L.scales, None, L.K, L.N, L.G, bias=L.bias)
    compare(y.cpu().numpy(), yD, A, f"symmetric M={M}")
    ref = oracle.dequant16(L.qweight, None, L.scales, None, L.K, L.N, L.G)
    for path in (q4.PATH_GEMV, q4.PATH_MFMA):
        assert np.array_equal(W.dequant_dump(path).cpu().numpy().view(np.uint16), ref)
    # fused: [symmetric part | stored-zero part]
    L2 = _layer(1024, 64, 128, M, 32)
    t2 = device_tensors(L2)
    Wc = q4.Q4Matrix.concat([(t["qweight"], None, t["scales"]),
                             (t2["qweight"], t2["qzeros"], t2["scales"])], groupsize=128)
    yc = Wc.matmul(t["x"])
    torch.cuda.synchronize()
    y1, A1 = oracle.matmul(L.x, L.qweight, None, L.scales, None, L.K, L.N, L.G)
    y2, A2 = oracle.matmul(L.x, L2.qweight, L2.qzeros, L2.scales, None, L.K, L2.N, L.G)
    compare(yc.cpu().numpy(), np.hstack([y1, y2]), np.hstack([A1, A2]), f"symmetric fused M={M}")


# ------------------------------------------------------------ HIP graphs --

@pytest.mark.parametrize("M,splits,act", [(1, 4, False), (3, 0, True), (40, 0, False), (64, 0, True)])
def test_graph_replay_matches_eager(M, splits, act):
    """q4_matmul captured in a HIP graph and replayed several times, with the
    program's own eager work and synchronizations between replays, gives the
    eager result every time: the split-K arrival counters are reset by the
    kernel itself and nothing in the captured path is a memset node."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    L = _layer(2048, 328, 128, M, 40 + M, act_order=act, bias=True)
    announce(f"graph M={M} splits={splits} act={act}")
    t = device_tensors(L)
    W = make_matrix(L, t)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ref = W.matmul(t["x"], t["bias"], splits=splits, stream=s).clone()
    s.synchronize()
    out = torch.empty_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        W.matmul(t["x"], t["bias"], out=out, splits=splits, stream=torch.cuda.current_stream())
    for r in range(4):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {r}"
        # eager work between replays on the same handle
        W.matmul(t["x"], splits=splits)
        torch.cuda.synchronize()
    yD, A = oracle_full(L)
    compare(out.cpu().numpy(), yD, A, f"graph M={M}")
