"""GPU parity of the streaming GEMM's stream-K schedule (needs an MI355X).

The workgroups of a stream-K launch share the (output tile, 64-row k-step)
iterations evenly, so a tile's K range can be split between two or more
workgroups; the last to arrive adds the fp32 partial sums in k order. Every
output must stay within the acceptance rule of tests/gpu_util against the
oracle for any number of workgroups: fewer than the tiles, more, one per
k-step (every tile split between all of its k-steps' workgroups) and more
than there are iterations (reduced to one each). The reduction order depends only
on the schedule, so a repeated call gives the same bits, and one workgroup
per tile gives exactly the one-tile-per-workgroup result.
"""
import warnings

import numpy as np
import pytest

import synth
from tests.gpu_util import (BF16_GEMM_REL_A, BF16_REL_Y, REL_A, REL_Y, announce, compare,
                            device_tensors, make_matrix, oracle_full, to_float64, torch_mod)

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
    return synth.make_layer(K, N, G, M, seed=synth.layer_seed("streamk", K, N, G, M, seed), **kw)


def _tiles(M, N, waves=4):
    bm = 64 if M <= 512 else 256     # the tile height the library takes for M rows
    return -(-M // bm) * -(-N // (32 * waves))


SK_CASES = [
    # K, N, G, M, act, bias, xfmt, bits, workgroup counts
    # 256-row tiles: 15 tiles of 16 k-steps (240 iterations; the last row
    # tile holds 8 rows): 2..37 workgroups split tiles into 2..9 segments, 15
    # is one per tile, 240 gives every k-step its own workgroup, and 300
    # (more workgroups than iterations) is reduced to 240
    (1024, 520, 128, 520, False, True, "f16", 4, (2, 3, 7, 13, 15, 20, 37, 240, 300)),
    # groups of 32 and a K tail inside the last k-step: 6 tiles of 2 k-steps
    (96, 136, 32, 520, False, False, "f16", 4, (3, 5, 8)),
    # 8 row tiles: XCD-ordered spaces when the count divides by 8 (8, 16, 40, 96)
    (256, 264, 128, 2048, False, True, "f16", 4, (8, 12, 16, 24, 40, 96)),
    # act-order (permuted activations), 64-row tiles: 8 tiles of 16 k-steps
    (1024, 256, 128, 256, True, True, "f16", 4, (3, 5)),
    # bfloat16 activations and 8-bit weights
    (512, 264, 128, 520, False, True, "bf16", 4, (5, 11)),
    (512, 264, 64, 520, False, True, "f16", 8, (5, 11)),
    # groups of 32 and a K tail with bfloat16, and with 8-bit weights
    (480, 136, 32, 516, False, True, "bf16", 4, (3, 7)),
    (480, 136, 32, 516, True, True, "f16", 8, (3, 7)),
    # 64-row tiles (M <= 512): 5 tiles of 16 k-steps; 80 = one k-step each
    (1024, 520, 128, 40, False, True, "f16", 4, (2, 5, 9, 40, 80, 100)),
    (1024, 520, 128, 64, True, True, "f16", 4, (3, 13)),
    (480, 136, 32, 17, False, True, "bf16", 4, (3, 7)),
    (480, 136, 32, 33, True, False, "f16", 8, (3, 7)),
]


# The same with 256 x 256 tiles (eight waves a workgroup, variant 8; only
# with 256-row tiles): column tiles 256 wide with a ragged last one, a
# partial last row tile, K tails, groups of 32, act-order, bfloat16, 8-bit.
SK_WIDE_CASES = [
    # 3 x 3 tiles (N = 520: 256 + 256 + 8 columns) of 16 k-steps: 144 iterations
    (1024, 520, 128, 520, False, True, "f16", 4, (2, 3, 7, 9, 20, 144, 200)),
    # groups of 32 and a K tail: 3 tiles of 2 k-steps
    (96, 136, 32, 520, False, False, "f16", 4, (2, 5)),
    # 8 row tiles x 3 column tiles: XCD-ordered spaces when the count divides by 8
    (256, 600, 128, 2048, False, True, "f16", 4, (8, 16, 24, 40)),
    (512, 520, 128, 520, True, True, "f16", 4, (5, 9)),
    (512, 520, 128, 520, False, True, "bf16", 4, (5, 11)),
    (512, 520, 64, 520, False, True, "f16", 8, (5, 11)),
    (480, 264, 32, 516, True, True, "bf16", 4, (3, 7)),
    (480, 264, 32, 516, False, False, "f16", 8, (3, 7)),
]
SK_ALL = [c + (0,) for c in SK_CASES] + [c + (8,) for c in SK_WIDE_CASES]


@pytest.mark.parametrize("K,N,G,M,act,bias,xfmt,bits,workers,variant", SK_ALL)
def test_stream_k_parity(K, N, G, M, act, bias, xfmt, bits, workers, variant):
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    L = _layer(K, N, G, M, 0, act_order=act, bias=bias, xfmt=xfmt, bits=bits)
    t = device_tensors(L)
    W = make_matrix(L, t)
    yD, A = oracle_full(L)
    tol = (dict(rel_a=BF16_GEMM_REL_A, rel_y=BF16_REL_Y) if xfmt == "bf16"
           else dict(rel_a=REL_A, rel_y=REL_Y))
    waves = 8 if variant == 8 else 4
    if variant == 0:
        assert q4.plan_gemm_waves(M, N, K) == 4, "the narrow cases expect 128-column tiles planned"
    announce(f"stream-k K={K} N={N} G={G} M={M} act={act} {xfmt} w{bits} variant={variant} one-per-tile")
    one = W.matmul(t["x"], t["bias"], path=q4.PATH_MFMA, variant=variant, splits=1)
    torch.cuda.synchronize()
    compare(to_float64(one), yD, A, f"one per tile K={K} N={N} M={M}", **tol)
    for P in workers:
        announce(f"stream-k K={K} N={N} G={G} M={M} act={act} {xfmt} w{bits} variant={variant} workers={P}")
        a = W.matmul(t["x"], t["bias"], path=q4.PATH_MFMA, variant=variant, splits=P)
        b = W.matmul(t["x"], t["bias"], path=q4.PATH_MFMA, variant=variant, splits=P)
        torch.cuda.synchronize()
        compare(to_float64(a), yD, A, f"stream-k K={K} N={N} M={M} workers={P}", **tol)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"workers={P}: not repeatable"
        if P == _tiles(M, N, waves):
            assert torch.equal(a.view(torch.int16), one.view(torch.int16)), \
                f"workers={P}: one workgroup per tile should match splits=1"
        iters = _tiles(M, N, waves) * -(-K // 64)
        if P > iters:
            c = W.matmul(t["x"], t["bias"], path=q4.PATH_MFMA, variant=variant, splits=iters)
            torch.cuda.synchronize()
            assert torch.equal(a.view(torch.int16), c.view(torch.int16)), \
                f"workers={P} should run as {iters}"


@pytest.mark.parametrize("M,splits", [(33, 0), (33, 7), (40, 1), (63, 0), (65, 0), (100, 5), (520, 0), (520, 7)])
def test_partial_row_tile_stays_in_output(M, splits):
    """A partial last row tile (64-row tiles up to M = 512, 256-row above)
    drops its rows past M: written into the first M rows of a longer buffer,
    the output equals the exact-size call bit for bit and the rows after it
    keep their contents."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    K, N = 1024, 520
    L = _layer(K, N, 128, M, 4, bias=True)
    t = device_tensors(L)
    W = make_matrix(L, t)
    announce(f"partial row tile M={M} splits={splits}")
    ref = W.matmul(t["x"], t["bias"], path=q4.PATH_MFMA, splits=splits)
    big = torch.empty((M + 80, N), dtype=torch.float16, device="cuda")
    big.view(torch.int16).fill_(0x5A5A)
    W.matmul(t["x"], t["bias"], out=big[:M], path=q4.PATH_MFMA, splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(big[:M].view(torch.int16), ref.view(torch.int16))
    assert bool((big[M:].view(torch.int16) == 0x5A5A).all()), "a store landed past row M"


def test_stream_k_planned_matches_explicit():
    """The planned schedule (splits=0) is the one q4_plan_gemm names."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    # (25 tiles of 64 k-steps: the plan shares them among 100 workgroups)
    L = _layer(4096, 520, 128, 300, 1, bias=True)
    t = device_tensors(L)
    W = make_matrix(L, t)
    P = q4.plan_gemm(300, 520, 4096, torch.cuda.get_device_properties(0).multi_processor_count)
    assert P != _tiles(300, 520)
    announce(f"stream-k planned workers={P}")
    a = W.matmul(t["x"], t["bias"], path=q4.PATH_MFMA)
    b = W.matmul(t["x"], t["bias"], path=q4.PATH_MFMA, splits=P)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_wide_tiles_planned():
    """A product the plan gives 256 x 256 tiles (256 of them on 256 CUs: one
    workgroup each): the planned call equals the explicit eight-wave launch
    bit for bit, and it and the 128-column launch meet the acceptance rule
    on whole rows and columns through every tile."""
    import gptq_bit_weight_amd as q4
    from tests.gpu_util import check_output
    torch = torch_mod()
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    M, N, K = 2048, 32 * cu, 128
    assert q4.plan_gemm_waves(M, N, K, cu) == 8
    L = _layer(K, N, 128, M, 3, bias=True)
    t = device_tensors(L)
    W = make_matrix(L, t)
    P = q4.plan_gemm(M, N, K, cu)
    announce(f"wide tiles planned M={M} N={N} K={K} workers={P}")
    a = W.matmul(t["x"], t["bias"], path=q4.PATH_MFMA)
    b = W.matmul(t["x"], t["bias"], path=q4.PATH_MFMA, variant=8, splits=P)
    c = W.matmul(t["x"], t["bias"], path=q4.PATH_MFMA, variant=4)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    check_output(L, a.cpu().numpy(), "wide tiles planned", seed=1)
    check_output(L, c.cpu().numpy(), "narrow tiles", seed=2)
    with pytest.raises(ValueError, match="variant 8"):
        W.matmul(t["x"][:512].contiguous(), path=q4.PATH_MFMA, variant=8)


def test_stream_k_graph_replay():
    """Captured stream-K launches replay with the eager result every time
    (the arrival counters are reset by the kernel), with other eager calls on
    the same handle in between; an explicit count whose workspace does not
    exist yet is refused under capture instead of allocating."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    L = _layer(1024, 520, 128, 300, 2, bias=True)
    t = device_tensors(L)
    W = make_matrix(L, t)
    s = torch.cuda.Stream()
    announce("stream-k graph eager reference")
    with torch.cuda.stream(s):
        ref = W.matmul(t["x"], t["bias"], splits=13, stream=s).clone()
    s.synchronize()
    out = torch.empty_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        W.matmul(t["x"], t["bias"], out=out, splits=13, stream=torch.cuda.current_stream())
    for r in range(4):
        announce(f"stream-k graph replay {r}")
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {r}"
        W.matmul(t["x"], splits=7)
        torch.cuda.synchronize()
    # 2048 rows: 40 tiles of 16 k-steps, so 1024 workgroups run as 640, more
    # than the stream's workspace was made for (2 x CUs)
    announce("stream-k capture refusal")
    x2 = torch.zeros((2048, 1024), dtype=torch.float16, device="cuda")
    out2 = torch.empty((2048, 520), dtype=torch.float16, device="cuda")
    g2 = torch.cuda.CUDAGraph()
    # (the refused call enqueues nothing, so torch warns that the graph is empty)
    with warnings.catch_warnings():
        warnings.filterwarnings("ignore", message="The CUDA Graph is empty")
        with torch.cuda.graph(g2, stream=s):
            with pytest.raises(ValueError, match="stream capture"):
                W.matmul(x2, out=out2, splits=q4.GEMM_MAX_WORKERS, stream=torch.cuda.current_stream())
    yD, A = oracle_full(L)
    compare(out.cpu().numpy(), yD, A, "stream-k graph")
