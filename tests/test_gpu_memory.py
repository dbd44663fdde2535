"""Device memory held by handles, and the stream-K workspace per stream
(needs an MI355X).

 - A Llama-7B-shaped block of handles (the seven layers at groupsize 128),
   used at every M the skinny kernel serves, holds at most 1.1 times the
   checkpoint bytes of its layers (packed weights + scales + packed zeros),
   measured as the drop in free device memory (so the device allocator's
   2 MiB rounding counts): the private layout is the packed size, the
   scale|zero words add 4 bytes per group column, and the split-K workspace
   is sized by the launch plan (none for most layers).
 - GEMM calls with the stream-K schedule on two streams at once, on separate
   handles, give the results each gives alone, bit for bit: every stream has
   its own partial-sum workspace and arrival counters.
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import announce, device_tensors, make_matrix, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_bit_weight_amd as q4
    q4.load_library()
    yield
    torch.cuda.empty_cache()


def test_block_of_handles_memory():
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    # a first handle on the device sets up the library's static workspace,
    # which is per GPU and not part of any handle
    tiny = synth.make_layer(512, 512, 128, 1, seed=1)
    make_matrix(tiny).close()
    layers, dev, metric = [], [], 0
    for name, K, N, bias in synth.LLAMA7B_BLOCK:
        L = synth.make_layer(K, N, 128, q4.GEMV_MAX_M, seed=synth.layer_seed("memory", name), bias=bias)
        layers.append(L)
        dev.append(device_tensors(L))
        metric += L.metric_bytes()
    outs = [torch.empty((q4.GEMV_MAX_M, L.N), dtype=torch.float16, device="cuda") for L in layers]
    xs = {M: [t["x"][:M].contiguous() for t in dev] for M in (1, 16, q4.GEMV_MAX_M)}
    # a first set of handles, used at the same M, loads the kernels' code
    # (the runtime places each code object in device memory on its first
    # launch); it stays alive so that no freed memory is reused below
    warm = [make_matrix(L, t) for L, t in zip(layers, dev)]
    for M in (1, 16, q4.GEMV_MAX_M):
        for W, x, o in zip(warm, xs[M], outs):
            W.matmul(x, out=o[:M])
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    announce("memory: 7B block of handles")
    mats = []
    for L, t in zip(layers, dev):
        before = torch.cuda.mem_get_info()[0]
        mats.append(make_matrix(L, t))
        torch.cuda.synchronize()
        announce(f"  {L.K}x{L.N}: {before - torch.cuda.mem_get_info()[0]} bytes for {L.metric_bytes()}")
    for M in (1, 16, q4.GEMV_MAX_M):
        for W, x, o in zip(mats, xs[M], outs):
            assert W.path_for(M) == q4.PATH_GEMV
            W.matmul(x, out=o[:M])
    torch.cuda.synchronize()
    held = free0 - torch.cuda.mem_get_info()[0]
    for W in mats + warm:
        W.close()
    announce(f"  handles hold {held} bytes for {metric} checkpoint bytes ({held / metric:.3f}x)")
    assert held <= 1.1 * metric, f"{held} bytes held for {metric} checkpoint bytes ({held / metric:.3f}x)"


def test_stream_k_on_two_streams():
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    La = synth.make_layer(1024, 520, 128, 300, seed=synth.layer_seed("two_streams", 0), bias=True)
    Lb = synth.make_layer(2048, 264, 128, 300, seed=synth.layer_seed("two_streams", 1))
    ta, tb = device_tensors(La), device_tensors(Lb)
    Wa, Wb = make_matrix(La, ta), make_matrix(Lb, tb)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    announce("stream-k two streams: references")
    ra = Wa.matmul(ta["x"], ta["bias"], splits=13)
    rb = Wb.matmul(tb["x"], splits=17)
    torch.cuda.synchronize()
    # first calls on each stream make their workspaces, outside the timed mix
    with torch.cuda.stream(sa):
        Wa.matmul(ta["x"], ta["bias"], splits=13, stream=sa)
    with torch.cuda.stream(sb):
        Wb.matmul(tb["x"], splits=17, stream=sb)
    torch.cuda.synchronize()
    announce("stream-k two streams: concurrent")
    oa = [torch.empty_like(ra) for _ in range(8)]
    ob = [torch.empty_like(rb) for _ in range(8)]
    for i in range(8):
        Wa.matmul(ta["x"], ta["bias"], out=oa[i], splits=13, stream=sa)
        Wb.matmul(tb["x"], out=ob[i], splits=17, stream=sb)
    torch.cuda.synchronize()
    for i in range(8):
        assert torch.equal(oa[i].view(torch.int16), ra.view(torch.int16)), f"stream a, call {i}"
        assert torch.equal(ob[i].view(torch.int16), rb.view(torch.int16)), f"stream b, call {i}"
    assert np.isfinite(ra.cpu().numpy()).all()
    Wa.close()
    Wb.close()
