"""A seeded sweep of mixed configurations against the oracle, every output
element (needs an MI355X).

The fixed cases elsewhere take one parameter at a time; here each case draws
all of them together from a seeded generator: K (a multiple of 32, often not
of 64 or 128), N (a multiple of 8, often not of 16), the group size (32, 64,
128, 256 or one group over K), M (1 ... 40, or 65 ... 600 on the GEMM),
act-order, bias, 4- or 8-bit codes, fp16 or bfloat16 activations, and the
path (automatic, or forced to the skinny kernel or to the GEMM). Each result
is checked element by element under the acceptance rule of its arithmetic
(tests/gpu_util.py), and a second call must give the same bits.
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import (BF16_GEMM_REL_A, BF16_REL_Y, REL_A, REL_Y, announce, compare, device_tensors,
                            make_matrix, oracle_full, run, to_float64, torch_mod)

pytestmark = pytest.mark.gpu

N_CASES = 40
MAX_MACS = 120_000_000     # keeps each oracle run short


def _draw(i):
    rng = np.random.default_rng(synth.layer_seed("sweep", i))
    while True:
        K = 32 * int(rng.integers(1, 97))             # 32 ... 3072
        N = 8 * int(rng.integers(1, 76))              # 8 ... 600
        G = int(rng.choice([32, 64, 128, 256, -1]))
        if G > 0 and K % G:
            continue
        M = int(rng.integers(1, 41)) if rng.random() < 0.7 else int(rng.integers(65, 601))
        if M * K * N > MAX_MACS:
            continue
        bits = 8 if rng.random() < 0.25 else 4
        if bits == 8 and N % 4:
            continue
        act = bool(G > 0 and K // G > 1 and rng.random() < 0.3)
        xfmt = "bf16" if rng.random() < 0.3 else "f16"
        bias = bool(rng.random() < 0.5)
        r = rng.random()
        path = 0 if r < 0.6 else (1 if (r < 0.8 and M <= 32) else 2)
        return dict(K=K, N=N, G=G, M=M, bits=bits, act=act, xfmt=xfmt, bias=bias, path=path)


CASES = [_draw(i) for i in range(N_CASES)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_bit_weight_amd as q4
    q4.load_library()
    yield
    torch.cuda.empty_cache()


@pytest.mark.parametrize("i", range(N_CASES), ids=[
    "K{K}_N{N}_G{G}_M{M}_b{bits}_{xfmt}{a}{b}_p{path}".format(a="_act" if c["act"] else "",
                                                          b="_bias" if c["bias"] else "", **c)
    for c in CASES])
def test_sweep_case(i):
    import gptq_bit_weight_amd as q4
    c = CASES[i]
    G = c["G"] if c["G"] > 0 else c["K"]
    L = synth.make_layer(c["K"], c["N"], G, c["M"], seed=synth.layer_seed("sweep-layer", i),
                         act_order=c["act"], bias=c["bias"], xfmt=c["xfmt"], bits=c["bits"])
    announce(f"sweep case {i}: {c}")
    t = device_tensors(L)
    W = make_matrix(L, t)
    taken = W.path_for(c["M"]) if c["path"] == 0 else c["path"]
    y = run(L, path=c["path"], W=W, t=t)
    y2 = run(L, path=c["path"], W=W, t=t)
    assert np.array_equal(np.asarray(y).view(np.uint8), np.asarray(y2).view(np.uint8)), "second call differs"
    yD, A = oracle_full(L)
    if c["xfmt"] == "bf16":
        rel_a = BF16_GEMM_REL_A if taken == q4.PATH_MFMA else REL_A
        compare(y, yD, A, f"sweep case {i}", rel_a=rel_a, rel_y=BF16_REL_Y)
    else:
        compare(y, yD, A, f"sweep case {i}", rel_a=REL_A, rel_y=REL_Y)
    W.close()
