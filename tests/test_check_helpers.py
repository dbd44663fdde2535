"""The parity checkers themselves (CPU only): the whole-row / whole-column
check used for GPU outputs with M > 16 must reach every output tile, and a
wrong value over any one wave's part of a tile (the GEMM's waves each own
32 columns of a 64- or 256-row tile) must fail it. The "GPU output" here is
the oracle's own result rounded to fp16, with a mistake planted in it.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util


@pytest.fixture(scope="module")
def layer_and_y():
    L = synth.make_layer(512, 392, 128, 600, seed=synth.layer_seed("check_helpers"))
    yD, A = gpu_util.oracle_full(L)
    return L, oracle.half_to_double(oracle.double_to_half(yD)), yD, A


def test_clean_output_passes(layer_and_y):
    L, y, _, _ = layer_and_y
    n = gpu_util.check_rows_cols(L, y, "clean")
    assert 0 < n < L.M * L.N


@pytest.mark.parametrize("M", [17, 200, 600, 2048])
def test_every_tile_is_reached(M):
    """Whole rows reach every row tile of the GEMM (64 rows up to M = 512,
    else 256) and whole columns every 128-column tile."""
    bm = 64 if M <= 512 else 256
    rows = gpu_util.tile_lines(M, bm, 1, 1, first=True)
    cols = np.unique(np.concatenate([[0], gpu_util.tile_lines(11008, 128, 1, 2)]))
    for r0 in range(0, M, bm):
        sel = rows[(rows >= r0) & (rows < r0 + bm)]
        assert min(r0 + bm, M) - 1 in sel and sel.size >= min(2, min(r0 + bm, M) - r0)
    for c0 in range(0, 11008, 128):
        assert ((cols >= c0) & (cols < c0 + 128)).any()


@pytest.mark.parametrize("r0,c0", [(0, 0), (256, 128), (512, 384), (256, 352)])
def test_planted_stripe_error_is_caught(layer_and_y, r0, c0):
    """A wrong value over one wave's 32 columns of one 256-row tile."""
    L, y, _, _ = layer_and_y
    bad = y.copy()
    bad[r0:r0 + 256, c0:c0 + 32] += 0.25
    with pytest.raises(AssertionError, match="outside tolerance"):
        gpu_util.check_rows_cols(L, bad, "planted")


def test_full_check_catches_single_element(layer_and_y):
    L, y, _, _ = layer_and_y
    small = synth.make_layer(256, 64, 128, 3, seed=7)
    yD, _ = gpu_util.oracle_full(small)
    ys = oracle.half_to_double(oracle.double_to_half(yD))
    assert gpu_util.check_output(small, ys, "clean") == ys.size
    ys[2, 63] += 0.05
    with pytest.raises(AssertionError, match="1 of 192"):
        gpu_util.check_output(small, ys, "one element")
