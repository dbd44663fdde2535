"""The allocation-free entry point q4_matmul_static (needs an MI355X).

It is q4_matmul_bias with every workspace taken from the library's static
per-GPU array. Checked here, through the C ABI:
 - two calls in a row on each handle, the second with fewer rows, each
   against q4_matmul_bias on the same inputs: bit for bit where both take
   the same launch plan (the skinny kernel, split or not, act-order staged in
   LDS or permuted into the array, and the GEMM with 64-row tiles), and
   within the acceptance rule against the oracle everywhere (the 256-row
   GEMM at M = 2048 may run fewer stream-K workgroups than planned);
 - no device memory is allocated by the calls (free device memory is the
   same before and after them; the array itself is placed when the handle
   is made);
 - captured into a graph, replays give the eager result;
 - act-order activations larger than the array are refused with
   NotImplementedError and the output is left untouched.
"""
import ctypes

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
    import gptq_bit_weight_amd as q4
    q4.load_library()
    yield


def _static(lib, W, x, bias, out, stream):
    st = lib.q4_matmul_static(W._h, ctypes.c_void_p(x.data_ptr()),
                              ctypes.c_void_p(bias.data_ptr()) if bias is not None else None,
                              ctypes.c_void_p(out.data_ptr()), int(x.shape[0]),
                              ctypes.c_void_p(stream.cuda_stream))
    return st


def _bias_call(lib, W, x, bias, out, stream):
    st = lib.q4_matmul_bias(W._h, ctypes.c_void_p(x.data_ptr()),
                            ctypes.c_void_p(bias.data_ptr()) if bias is not None else None,
                            ctypes.c_void_p(out.data_ptr()), int(x.shape[0]),
                            ctypes.c_void_p(stream.cuda_stream))
    return st


# K, N, G, M first call, M second call, act-order, bias, same plan as q4_matmul_bias
CASES = [
    (4096, 4096, 128, 1, 1, False, True, True),        # skinny kernel, unsplit
    (11008, 4096, 128, 8, 5, False, False, True),      # skinny kernel, K split in two
    (4096, 11008, 128, 4, 3, True, False, True),       # act-order: x[:, perm] in the array
    (4096, 11008, 128, 2, 1, True, True, True),        # act-order staged in LDS
    (4096, 11008, 128, 300, 40, False, True, True),    # GEMM, 64-row tiles, stream-K
    (11008, 4096, 128, 2048, 1024, False, False, False),   # 256-row stream-K: fewer workgroups
    (4096, 11008, 128, 2048, 600, True, True, False),  # act-order GEMM: x' and partials
]


@pytest.mark.parametrize("K,N,G,M1,M2,act,bias,same", CASES)
def test_static_matches_allocating_entry_point(K, N, G, M1, M2, act, bias, same):
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    lib = q4.load_library()
    L = synth.make_layer(K, N, G, M1, seed=synth.layer_seed("static", K, N, M1, act), act_order=act,
                         bias=bias)
    t = device_tensors(L)
    W = make_matrix(L, t)
    s = torch.cuda.Stream()
    outs = {}
    for M in (M1, M2):
        x = t["x"][:M].contiguous()
        outs[M] = (torch.empty((M, N), dtype=torch.float16, device="cuda"),
                   torch.empty((M, N), dtype=torch.float16, device="cuda"))
    # reference calls first (they allocate their own workspaces)
    for M in (M1, M2):
        announce(f"static ref K={K} N={N} M={M} act={act}")
        assert _bias_call(lib, W, t["x"][:M].contiguous(), t["bias"], outs[M][0], s) == 0, \
            lib.q4_last_error()
    s.synchronize()
    xs = {M: t["x"][:M].contiguous() for M in (M1, M2)}
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for M in (M1, M2):
        announce(f"static K={K} N={N} M={M} act={act}")
        st = _static(lib, W, xs[M], t["bias"], outs[M][1], s)
        assert st == 0, lib.q4_last_error()
    s.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert free1 == free0, f"device memory changed by {free0 - free1} bytes"
    for M in (M1, M2):
        ref, got = outs[M]
        if same:
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"M={M}: differs from q4_matmul_bias"
        Lm = synth.Layer(K=L.K, N=L.N, G=L.G, qweight=L.qweight, qzeros=L.qzeros, scales=L.scales,
                         g_idx=L.g_idx, x=L.x[:M], bias=L.bias, seed=L.seed)
        y = got.cpu().numpy()
        assert np.isfinite(y).all()
        check_output(Lm, y, f"static K={K} N={N} M={M}", seed=M)
    W.close()


def test_static_graph_replay():
    """Captured static calls (a split skinny launch, whose counters live in
    the array) replay with the eager result, with eager static calls on
    another handle in between."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    L = synth.make_layer(11008, 4096, 128, 8, seed=synth.layer_seed("static_graph"), bias=True)
    L2 = synth.make_layer(4096, 11008, 128, 4, seed=synth.layer_seed("static_graph2"), act_order=True)
    t, t2 = device_tensors(L), device_tensors(L2)
    W, W2 = make_matrix(L, t), make_matrix(L2, t2)
    s = torch.cuda.Stream()
    announce("static graph eager reference")
    with torch.cuda.stream(s):
        ref = W.matmul_static(t["x"], t["bias"], stream=s).clone()
        ref2 = W2.matmul_static(t2["x"], stream=s).clone()
    s.synchronize()
    out = torch.empty_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        W.matmul_static(t["x"], t["bias"], out=out, stream=torch.cuda.current_stream())
    for r in range(3):
        announce(f"static graph replay {r}")
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {r}"
        y2 = W2.matmul_static(t2["x"])
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int16), ref2.view(torch.int16)), f"eager between replays {r}"
    W.close()
    W2.close()


def test_static_refuses_oversized_act_order():
    """An act-order layer whose permuted activations exceed the array is
    refused before anything runs; smaller M on the same handle works."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    K, N = 28672, 1024
    L = synth.make_layer(K, N, 128, 1, seed=synth.layer_seed("static_big"), act_order=True)
    t = device_tensors(L)
    W = make_matrix(L, t)
    M = (q4.STATIC_SCRATCH_BYTES - (64 << 10)) // (2 * K) + 1
    x = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    out = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    announce(f"static oversized act-order M={M}")
    with pytest.raises(NotImplementedError, match="static workspace"):
        W.matmul_static(x, out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    y = W.matmul_static(x[:M - 1].contiguous())
    torch.cuda.synchronize()
    assert bool((y == 0).all())
    W.close()
