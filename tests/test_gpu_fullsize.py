"""GPU parity at the full workload sizes (needs an MI355X), in the launch
configuration the benchmark times (automatic path and split plan).

Every output element is held to the acceptance rule when M <= 32 (the
oracle computes the whole product: the 7B block, the act-order layers,
every M of the 70B sweep and the small batches the skinny kernel serves).
For M > 32 (prefill and larger small batches, on the GEMM) the oracle
computes whole output rows and whole output columns: for each 64-row stretch
its last row and a random one, for each 128-column stretch its first, last
and a random column, so every output tile and every stream-K split of it has
checked rows and columns. All outputs are also checked for run-to-run bit
identity and finiteness.

Workloads (shapes only, synthetic values): a Llama-7B-shaped decoder block
at M = 1 (q/k/v/o 4096x4096, gate/up 4096x11008, down 11008x4096, bias on
q), its act-order variant (4096x11008 and 11008x4096, M in {1, 4}), the
Llama-70B-shaped MLP (8192x28672 and 28672x8192, M in {1, 2, 4, 8, 16}),
prefill at M = 2048 (4096x11008 and 11008x4096, groupsize 128 and 32, plus
act-order) and small batches (M in {17, 32} on the skinny kernel's two row
blocks; 64, 200, 400, 600 on the GEMM).
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import announce, check_output, device_tensors, make_matrix, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.empty_cache()


def _check_layer(L, name):
    torch = torch_mod()
    announce(f"full-size {name} K={L.K} N={L.N} G={L.G} M={L.M} act={L.g_idx is not None}")
    t = device_tensors(L)
    W = make_matrix(L, t)
    y1 = W.matmul(t["x"], t["bias"])
    y2 = W.matmul(t["x"], t["bias"])
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "run-to-run difference"
    W.close()
    y = y1.cpu().numpy()
    assert np.isfinite(y).all()
    n = check_output(L, y, f"{name} M={L.M}", seed=L.seed)
    announce(f"  {n} of {y.size} elements checked against the oracle")


@pytest.mark.parametrize("layer", synth.LLAMA7B_BLOCK, ids=[l[0] for l in synth.LLAMA7B_BLOCK])
def test_llama7b_block_decode(layer):
    name, K, N, bias = layer
    L = synth.make_layer(K, N, 128, 1, seed=synth.layer_seed("llama7b_block_decode", name, 1),
                         bias=bias)
    _check_layer(L, name)


@pytest.mark.parametrize("K,N", [(4096, 11008), (11008, 4096)])
@pytest.mark.parametrize("M", [1, 4])
def test_llama7b_actorder(K, N, M):
    L = synth.make_layer(K, N, 128, M, seed=synth.layer_seed("llama7b_actorder", K, N, M),
                         act_order=True)
    _check_layer(L, f"act-order {K}x{N}")


@pytest.mark.parametrize("layer", synth.LLAMA70B_MLP, ids=[l[0] for l in synth.LLAMA70B_MLP])
@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_llama70b_mlp_decode(layer, M):
    name, K, N = layer
    L = synth.make_layer(K, N, 128, M, seed=synth.layer_seed("llama70b_mlp_decode", name, M))
    _check_layer(L, name)


@pytest.mark.parametrize("K,N,G,act", [(4096, 11008, 128, False), (11008, 4096, 128, False),
                                       (4096, 11008, 32, False), (11008, 4096, 32, False),
                                       (4096, 11008, 128, True)])
def test_prefill(K, N, G, act):
    L = synth.make_layer(K, N, G, 2048, seed=synth.layer_seed("prefill", K, N, G, act),
                         act_order=act)
    _check_layer(L, f"prefill {K}x{N} G{G}")


@pytest.mark.parametrize("K,N", [(4096, 11008), (11008, 4096), (28672, 8192)])
@pytest.mark.parametrize("M", [17, 32, 64, 200, 400, 600])
def test_small_batch(K, N, M):
    """Batches past 16 rows: the skinny kernel's two row blocks (M <= 32);
    then the GEMM's 64-row output tiles (M <= 512), with stream-K across the
    CUs; and 600 rows: three 256-row tiles."""
    L = synth.make_layer(K, N, 128, M, seed=synth.layer_seed("small_batch", K, N, M), bias=True)
    _check_layer(L, f"small batch {K}x{N}")


@pytest.mark.parametrize("K,N,M", [(4096, 4096, 3000), (4096, 11008, 4100), (4096, 11008, 1536)])
def test_long_prefill(K, N, M):
    """Longer prompts than the benchmark's: 3000 rows (11 full 256-row tiles
    and a 184-row one: 384 tiles on 512 stream-K workgroups), 4100 rows
    (17 x 86 tiles, one workgroup per tile, a 4-row last tile) and 1536 rows
    (516 tiles on 512 stream-K workgroups, nearly every tile split); whole
    rows and columns through every tile."""
    L = synth.make_layer(K, N, 128, M, seed=synth.layer_seed("long_prefill", K, N, M), bias=True)
    _check_layer(L, f"long prefill {K}x{N}")
