"""Host threads using the library at once (needs an MI355X).

Four threads each make their own handle (q4_make runs concurrently: device
synchronization, the per-device static set-up) and then, each on its own
stream, alternate skinny-kernel calls with K split over workgroups and GEMM
calls on the stream-K schedule (per-stream workspaces made on first use).
Every result must equal, bit for bit, the one the same handle gives when
called alone beforehand, and the references must match the oracle. The
library's host state (workspace maps, per-handle buffers, the thread-local
error) is behind its own locks; this exercises them from several threads.
"""
import threading

import numpy as np
import pytest

import synth
from tests.gpu_util import announce, compare, device_tensors, make_matrix, oracle_full, torch_mod

pytestmark = pytest.mark.gpu

SHAPES = [(1024, 520, 128), (2048, 264, 64), (1536, 392, 128), (512, 1032, 32)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_bit_weight_amd as q4
    q4.load_library()
    yield
    torch.cuda.empty_cache()


def test_threads_make_and_call_concurrently():
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    layers = [synth.make_layer(K, N, G, 300, seed=synth.layer_seed("threads", i), bias=(i % 2 == 0))
              for i, (K, N, G) in enumerate(SHAPES)]
    dev = [device_tensors(L) for L in layers]
    torch.cuda.synchronize()
    mats = [None] * len(layers)
    errors = []

    def make(i):
        try:
            mats[i] = make_matrix(layers[i], dev[i])
        except Exception as e:      # reported below, on the main thread
            errors.append(f"make {i}: {e!r}")

    announce("threads: concurrent q4_make")
    ts = [threading.Thread(target=make, args=(i,)) for i in range(len(layers))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors

    # references, one handle at a time: M = 8 with 4 K splits (skinny kernel)
    # and M = 300 with 24 workgroups (stream-K)
    announce("threads: references")
    refs = []
    for W, t in zip(mats, dev):
        a = W.matmul(t["x"][:8].contiguous(), t["bias"], path=q4.PATH_GEMV, splits=4)
        b = W.matmul(t["x"], t["bias"], path=q4.PATH_MFMA, splits=24)
        refs.append((a.clone(), b.clone()))
    torch.cuda.synchronize()
    for L, (a, b) in zip(layers, refs):
        yD, A = oracle_full(L)
        compare(b.cpu().numpy(), yD, A, f"threads reference {L.K}x{L.N}")
        compare(a.cpu().numpy(), yD[:8], A[:8], f"threads reference {L.K}x{L.N} M=8")

    outs = [[] for _ in layers]

    def work(i):
        try:
            s = torch.cuda.Stream()
            W, t = mats[i], dev[i]
            x8 = t["x"][:8].contiguous()
            with torch.cuda.stream(s):
                # (first calls on this stream make its stream-K workspace)
                for r in range(10):
                    a = W.matmul(x8, t["bias"], path=q4.PATH_GEMV, splits=4, stream=s)
                    b = W.matmul(t["x"], t["bias"], path=q4.PATH_MFMA, splits=24, stream=s)
                    outs[i].append((a, b))
            s.synchronize()
        except Exception as e:
            errors.append(f"thread {i}: {e!r}")

    announce("threads: concurrent calls")
    ts = [threading.Thread(target=work, args=(i,)) for i in range(len(layers))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (ra, rb) in enumerate(refs):
        assert len(outs[i]) == 10
        for r, (a, b) in enumerate(outs[i]):
            assert torch.equal(a.view(torch.int16), ra.view(torch.int16)), f"thread {i} call {r}: skinny kernel"
            assert torch.equal(b.view(torch.int16), rb.view(torch.int16)), f"thread {i} call {r}: GEMM"
    for W in mats:
        W.close()
