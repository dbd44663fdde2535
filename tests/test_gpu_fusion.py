"""Projection fusion on the GPU (q4_make_cat): one handle over the column
concatenation of layers that take the same input (GPTQModel wiki "Inference
Backends", section "How AUTO selection works": QKV and gate/up calls combined
after backend selection).

 - parity with the oracle on the concatenated layer, both kernels;
 - every column equals the result of its own part's handle bit for bit (same
   kernel, same accumulation order);
 - a shared act-order g_idx;
 - argument errors;
 - the Llama-7B-shaped q/k/v and gate/up stacks at full size (every element).
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import announce, check_output, compare, oracle_full, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_bit_weight_amd as q4
    q4.load_library()
    yield


def _parts(K, Ns, G, M, seed, act_order=False, bias=(True,)):
    parts = [synth.make_layer(K, n, G, M, seed=synth.layer_seed("fusion", K, n, G, M, seed, i),
                              act_order=act_order, bias=bias[i % len(bias)])
             for i, n in enumerate(Ns)]
    for p in parts[1:]:
        p.g_idx = parts[0].g_idx            # parts of one fused call share the input ordering
    return parts


def _dev(torch, a):
    return torch.from_numpy(a).to(torch.device("cuda", 0)) if a is not None else None


def _make(q4, torch, parts):
    dev_parts = [(_dev(torch, p.qweight), _dev(torch, p.qzeros), _dev(torch, p.scales)) for p in parts]
    return q4.Q4Matrix.concat(dev_parts, g_idx=_dev(torch, parts[0].g_idx), groupsize=parts[0].G)


@pytest.mark.parametrize("K,Ns,G,M,act", [
    (1024, (264, 136, 520), 128, 1, False),     # uneven widths, skinny kernel
    (1024, (264, 136, 520), 128, 5, False),
    (512, (64, 64, 64), 32, 16, False),         # groups of 32 at the skinny limit
    (768, (128, 200), 64, 33, False),           # GEMM path
    (1024, (96, 160), 128, 4, True),            # shared act-order g_idx
    (1024, (96, 160), 128, 70, True),
])
def test_fused_parity(K, Ns, G, M, act):
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    parts = _parts(K, Ns, G, M, 0, act_order=act, bias=(True, False))
    cat = synth.concat_layers(parts)
    announce(f"fused K={K} N={Ns} G={G} M={M} act={act}")
    W = _make(q4, torch, parts)
    assert W.N == sum(Ns) and W.part_n == tuple(Ns) and W.act_order == act
    x, b = _dev(torch, cat.x), _dev(torch, cat.bias)
    y = W.matmul(x, b)
    torch.cuda.synchronize()
    yD, A = oracle_full(cat)
    compare(y.cpu().numpy(), yD, A, f"fused K={K} N={Ns} M={M}")
    assert [tuple(v.shape) for v in W.split(y)] == [(M, n) for n in Ns]


@pytest.mark.parametrize("M,path", [(1, 1), (8, 1), (16, 1), (40, 2)])
def test_fused_columns_equal_part_handles(M, path):
    """Each column of the fused result is bit-identical to its part's own
    handle: the kernels treat columns independently and accumulate each in the
    same order (the skinny kernel is pinned to one column tile and no K split,
    the GEMM to one workgroup per output tile, so both handles take the same
    plan)."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    parts = _parts(2048, (256, 512, 128), 128, M, 1, bias=(False,))
    announce(f"fused vs parts M={M} path={path}")
    W = _make(q4, torch, parts)
    x = _dev(torch, parts[0].x)
    variant, splits = (1, 1) if path == 1 else (0, 1)
    y = W.matmul(x, path=path, variant=variant, splits=splits)
    singles = []
    for p in parts:
        Wp = q4.Q4Matrix(_dev(torch, p.qweight), _dev(torch, p.qzeros), _dev(torch, p.scales), None, 128)
        singles.append(Wp.matmul(x, path=path, variant=variant, splits=splits))
    torch.cuda.synchronize()
    for got, ref in zip(W.split(y), singles):
        assert torch.equal(got.contiguous().view(torch.int16), ref.view(torch.int16))


def test_fused_argument_errors():
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    a = synth.make_layer(256, 64, 128, 1, seed=5)
    b = synth.make_layer(512, 64, 128, 1, seed=6)
    announce("fused errors")
    pa = (_dev(torch, a.qweight), _dev(torch, a.qzeros), _dev(torch, a.scales))
    pb = (_dev(torch, b.qweight), _dev(torch, b.qzeros), _dev(torch, b.scales))
    with pytest.raises(ValueError, match="K="):
        q4.Q4Matrix.concat([pa, pb])
    with pytest.raises(ValueError):
        q4.Q4Matrix.concat([])
    W = q4.Q4Matrix.concat([pa, pa, pa])
    assert W.N == 192 and W.path_for(1) == q4.PATH_GEMV
    W.close()


@pytest.mark.parametrize("group", ["qkv_proj", "gate_up_proj"])
def test_llama7b_fused_full_size(group):
    """The fused q/k/v and gate/up stacks of the 7B block at M = 1 and 4,
    every element against the oracle, with the launch the benchmark uses
    (automatic plan)."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    names = dict(synth.LLAMA7B_FUSED)[group]
    spec = {n: (K, N, bias) for n, K, N, bias in synth.LLAMA7B_BLOCK}
    for M in (1, 4):
        parts = [synth.make_layer(spec[n][0], spec[n][1], 128, M,
                                  seed=synth.layer_seed("fusion_full", n, M), bias=spec[n][2])
                 for n in names]
        cat = synth.concat_layers(parts)
        announce(f"fused full {group} M={M} N={cat.N}")
        W = _make(q4, torch, parts)
        y = W.matmul(_dev(torch, cat.x), _dev(torch, cat.bias))
        torch.cuda.synchronize()
        W.close()
        check_output(cat, y.cpu().numpy(), f"{group} M={M}")
