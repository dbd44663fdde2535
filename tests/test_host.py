"""CPU-only tests of libq4: the library loads and exports every symbol the
header declares, and the host-side planning (argument checks, act-order
plan, split plan) behaves as documented. No GPU call is made here.

Passages: "Implementation: Predibase Lorax GPTQ Exllama V1", Description
(handle from qweight/qzeros/scales/g_idx; act-order detected by a non-trivial
g_idx) and I/O contract (bits = 4, groupsize); GPTQModel wiki "Inference
Backends", section "Runtime cache lifetime" (one stable argsort of g_idx;
identity permutation skips the gather).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import gptq_bit_weight_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "q4.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = q4.load_library()
    declared = _header_functions()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(lib, name), name                   # dlsym succeeds
    assert sorted(q4.EXPORTED_SYMBOLS) == declared


def test_library_links_only_hip_runtime():
    """The product library is self-contained HIP: it does not link torch or
    the CPU oracle."""
    import subprocess
    out = subprocess.run(["ldd", q4.library_path()], capture_output=True, text=True).stdout
    assert "libamdhip64" in out
    assert "torch" not in out and "oracle" not in out


def test_missing_library_raises(tmp_path, monkeypatch):
    monkeypatch.setattr(q4, "_lib", None)
    monkeypatch.setattr(q4, "_LIB_PATH", str(tmp_path / "libq4.so"))
    with pytest.raises(ImportError):
        q4.load_library()


@pytest.mark.parametrize("K,N,G", [(512, 512, 128), (4096, 11008, 128), (11008, 4096, 128),
                                   (8192, 28672, 128), (96, 8, 32), (256, 64, 64), (512, 8, 256),
                                   (96, 16, -1)])
def test_check_shape_accepts(K, N, G):
    q4.check_shape(K, N, G)


@pytest.mark.parametrize("K,N,G,exc", [
    (0, 512, 128, ValueError), (512, 0, 128, ValueError), (516, 512, 128, ValueError),
    (512, 516, 128, ValueError), (512, 512, 100, NotImplementedError),
    (512, 512, 0, NotImplementedError), (520, 512, -1, NotImplementedError),
    (384, 512, 256, NotImplementedError),
])
def test_check_shape_rejects(K, N, G, exc):
    with pytest.raises(exc):
        q4.check_shape(K, N, G)


def test_check_shape_message_names_the_problem():
    with pytest.raises(ValueError, match="multiple of 8"):
        q4.check_shape(512, 12, 128)


def test_plan_actorder_is_stable_argsort():
    rng = np.random.default_rng(0)
    K, G = 1024, 128
    pi = rng.permutation(K)
    pos = np.empty(K, dtype=np.int64)
    pos[pi] = np.arange(K)
    g = (pos // G).astype(np.int32)
    perm, trivial = q4.plan_actorder(g, K, G)
    assert not trivial
    assert np.array_equal(perm, np.argsort(g, kind="stable"))
    assert np.array_equal(g[perm], np.arange(K) // G)


def test_plan_actorder_trivial_is_identity():
    K, G = 512, 128
    g = (np.arange(K) // G).astype(np.int32)
    perm, trivial = q4.plan_actorder(g, K, G)
    assert trivial and np.array_equal(perm, np.arange(K))


def test_plan_actorder_ties_keep_k_order():
    K, G = 64, 32
    g = np.array([1, 0] * 32, dtype=np.int32)           # odd rows group 0, even rows group 1
    perm, trivial = q4.plan_actorder(g, K, G)
    assert not trivial
    assert perm.tolist() == list(range(1, 64, 2)) + list(range(0, 64, 2))


def test_plan_actorder_rejects_out_of_range_and_nonuniform():
    K, G = 128, 32
    g = (np.arange(K) // G).astype(np.int32)
    bad = g.copy()
    bad[5] = 4
    with pytest.raises(ValueError, match="outside"):
        q4.plan_actorder(bad, K, G)
    bad = g.copy()
    bad[5] = -1
    with pytest.raises(ValueError):
        q4.plan_actorder(bad, K, G)
    uneven = g.copy()
    uneven[0] = 1                                        # group 0: 31 rows, group 1: 33 rows
    with pytest.raises(NotImplementedError, match="not uniform"):
        q4.plan_actorder(uneven, K, G)


def test_plan_gemv():
    # column tiles in {1, 2, 4}, splits a power of 2 <= 16; splits only when the
    # column tiles cannot give every CU a workgroup
    for (M, K, N) in [(1, 4096, 4096), (1, 4096, 11008), (1, 11008, 4096), (1, 8192, 28672),
                      (16, 28672, 8192), (16, 8192, 28672), (1, 512, 512), (4, 96, 8)]:
        ct, s = q4.plan_gemv(M, K, N, 128 if K % 128 == 0 else 32, num_cu=256)
        assert ct in (1, 2, 4) and s in (1, 2, 4, 8, 16), (M, K, N, ct, s)
        tiles = -(-N // (16 * ct))
        assert s == 1 or tiles * s <= 256, (M, K, N, ct, s)
    assert q4.plan_gemv(1, 4096, 4096, 128, num_cu=256) == (1, 1)       # 256 tiles of 16
    assert q4.plan_gemv(16, 4096, 4096, 128, num_cu=256) == (1, 1)      # wider: half the CUs idle
    assert q4.plan_gemv(1, 4096, 11008, 128, num_cu=256) == (1, 1)      # 688 tiles fill 3 rounds
    assert q4.plan_gemv(8, 4096, 11008, 128, num_cu=256) == (4, 1)      # reuse wins with 8 rows
    assert q4.plan_gemv(1, 28672, 8192, 128, num_cu=256) == (2, 1)      # 256 tiles of 32
    assert q4.plan_gemv(1, 8192, 28672, 128, num_cu=256) == (1, 1)      # 1792 tiles fill 7 rounds
    assert q4.plan_gemv(1, 4096, 22016, 128, num_cu=256) == (1, 1)      # 1376 tiles: finer last round
    assert q4.plan_gemv(1, 4096, 12288, 128, num_cu=256) == (1, 1)      # 768 tiles fill 3 rounds
    assert q4.plan_gemv(4, 8192, 28672, 128, num_cu=256) == (4, 1)
    assert q4.plan_gemv(16, 8192, 28672, 32, num_cu=256)[0] == 2        # groups of 32: at most 2
    assert q4.plan_gemv(1, 4096, 1024, 128, num_cu=256) == (1, 4)       # 64 tiles, 32 blocks
    # M > 4 on narrow layers: wide tiles split in K while waves keep 4 blocks
    assert q4.plan_gemv(16, 28672, 8192, 128, num_cu=256) == (4, 2)
    assert q4.plan_gemv(8, 28672, 8192, 128, num_cu=256) == (4, 2)
    assert q4.plan_gemv(16, 11008, 4096, 128, num_cu=256) == (2, 2)
    assert q4.plan_gemv(8, 11008, 4096, 128, num_cu=256) == (2, 2)
    assert q4.plan_gemv(8, 4096, 4096, 128, num_cu=256) == (1, 1)       # 32 blocks: no split
    assert q4.plan_gemv(4, 28672, 8192, 128, num_cu=256) == (2, 1)      # M <= 4: splits cost more
    assert q4.plan_gemv(1, 512, 512, 128, num_cu=256) == (1, 1)         # 4 blocks: too few to split
    with pytest.raises(ValueError):
        q4.plan_gemv(0, 4096, 4096, 128)
    with pytest.raises(ValueError):
        q4.plan_gemv(q4.GEMV_MAX_M + 1, 4096, 4096, 128)
    # two row blocks (16 < M <= 32)
    for M in (17, 32):
        for K, N, G in ((4096, 4096, 128), (4096, 11008, 128), (11008, 4096, 128), (4096, 11008, 32)):
            ct, s = q4.plan_gemv(M, K, N, G, num_cu=256)
            assert ct in ((1, 2) if G == 32 else (1, 2, 4)), (M, K, N, G, ct)
            assert s in (1, 2, 4, 8, 16)
    with pytest.raises(NotImplementedError):
        q4.plan_gemv(1, 4128, 4096, 128)      # K % groupsize != 0


def test_plan_gemm():
    """At the planned tile width (q4_plan_gemm_waves). 128-column tiles (four
    waves, two workgroups per CU): one workgroup per output tile (256 x 128,
    or 64 x 128 for M <= 512) when the tiles fill whole rounds of two per CU
    (to within a tenth) or make 1.5 rounds or more; otherwise the workgroups
    share the k-steps (stream-K): for 64-row tiles 2 x CUs workgroups from
    32 k-steps each, CUs from 16, else 16 k-steps each (at least one per
    tile); for 256-row ones min(2 CUs, max(2 tiles, CUs)). 256 x 256 tiles
    (eight waves, one workgroup per CU): one per tile when the tiles fill
    whole rounds of CUs to within a tenth, else one round of CUs sharing the
    k-steps. Never more than there are (tile, 64-row k-step) iterations."""
    p = q4.plan_gemm
    assert p(2048, 4096, 11008, 256) == 256      # 128 wide tiles, 172 k-steps: one round of CUs
    assert p(2048, 11008, 4096, 256) == 256      # 344 wide tiles: 1.34 rounds
    assert p(2048, 12288, 4096, 256) == 256      # fused q/k/v: 384 wide tiles, 1.5 rounds
    assert p(4096, 4096, 4096, 256) == 256       # 256 wide tiles: one whole round
    assert p(16384, 28672, 8192, 256) == 7168    # 28 whole rounds of wide tiles
    assert p(2048, 28672, 8192, 256) == 256      # 896 wide tiles: 3.5 rounds
    assert p(2048, 8192, 128, 256) == 256        # 256 wide tiles of 2 k-steps: one per tile
    assert p(2048, 4096, 4096, 256) == 512       # 128 wide tiles, 32 k-steps a CU: narrow, 256 tiles
    assert p(17, 4096, 4096, 256) == 128         # 64-row tiles: 2048 iterations, 16 a workgroup
    assert p(64, 4096, 11008, 256) == 256        # 5504 iterations: 21.5 each on one a CU
    assert p(32, 28672, 8192, 256) == 512        # 28672: 56 each on two a CU
    assert p(64, 11008, 4096, 256) == 256
    assert p(128, 11008, 4096, 256) == 256       # 2 x 86 tiles x 64 k-steps: 21.5 each at 2 a CU, too few
    assert p(256, 4096, 4096, 256) == 256        # 8192 iterations: 32 each on one a CU, 16 at two
    assert p(64, 1024, 1024, 256) == 8           # 8 tiles x 16 k-steps: one per tile
    assert p(256, 4096, 11008, 256) == 512       # 4 x 32 tiles x 172 k-steps: at most 2 x CUs
    assert p(512, 4096, 11008, 256) == 512       # 8 x 32 tiles of 64 rows x 172 k-steps: 2 x CUs
    assert p(520, 6144, 4096, 256) == 288        # 3 x 48 tiles of 256 rows: 2 x tiles
    assert p(520, 4096, 11008, 256) == 256       # 3 x 32 tiles of 256 rows: at least one per CU
    assert p(520, 136, 96, 256) == 12            # 6 tiles of 2 k-steps: 12 iterations
    assert p(520, 136, 32, 256) == 6             # 6 tiles of 1 k-step: one each
    assert p(2048, 4096, 11008, 64) == 128       # a smaller chip: 128 wide tiles, two whole rounds
    assert p(2048, 11008, 4096, 64) == 64        # 344 wide tiles: 5.4 rounds of 64, stream-K
    for bad in ((0, 8, 32), (1, 0, 32), (1, 8, 0)):
        with pytest.raises(ValueError):
            p(*bad)


def test_plan_gemm_waves():
    """256-column tiles (eight waves) only with 256-row tiles (M > 512), when
    the 256 x 256 tiles are at least the CUs, or half of them with at least
    64 (tile, k-step) pairs a CU, or any number with at least 128 a CU."""
    w = q4.plan_gemm_waves
    assert w(512, 28672, 8192, 256) == 4         # 64-row tiles: always four
    assert w(1536, 11008, 4096, 256) == 8        # 6 x 43 = 258 tiles
    assert w(1024, 11008, 4096, 256) == 4        # 172 tiles, 43 pairs a CU
    assert w(2048, 4096, 11008, 256) == 8        # 128 tiles, 86 pairs a CU
    assert w(1536, 4096, 11008, 256) == 4        # 96 tiles, 64 pairs a CU
    assert w(2048, 4096, 4096, 256) == 4         # 128 tiles, 32 pairs a CU
    assert w(4096, 4096, 4096, 256) == 8         # 256 tiles
    assert w(768, 8192, 28672, 256) == 8         # 96 tiles, 168 pairs a CU
    assert w(520, 136, 96, 256) == 4
    for bad in ((0, 8, 32), (1, 0, 32), (1, 8, 0)):
        with pytest.raises(ValueError):
            w(*bad)


def test_plan_gemv_gather():
    """Act-order activations are staged by the skinny kernel itself only when
    K is not split, M <= 2, K padded to whole blocks is at most 12288 rows and
    M rows of it (8 halfs of padding each) fit 20480 halfs; otherwise a
    separate permute runs."""
    g = q4.plan_gemv_gather
    assert g(1, 4096, 1) and g(2, 4096, 1)              # 7B gate/up at M = 1, 2
    assert not g(3, 4096, 1) and not g(4, 1024, 1)      # M > 2: separate permute
    assert g(1, 11008, 1)                               # 7B down at M = 1: 11008 rows
    assert not g(2, 11008, 1)                           # 2 x 11016 halfs > 20480
    assert g(2, 10112, 1) and not g(2, 10240, 1)        # 2 x 10120 fits, 2 x 10248 does not
    assert not g(1, 4096, 2)                            # split K
    assert not g(1, 12416, 1) and g(1, 12288, 1)        # 97 blocks exceed 12288 rows
    assert g(1, 12200, 1)                               # 96 blocks once padded
    for bad in ((0, 4096, 1), (q4.GEMV_MAX_M + 1, 4096, 1), (1, 4096, 0), (1, 4096, 17), (1, 0, 1)):
        with pytest.raises(ValueError):
            g(*bad)


def test_check_shape_size_limit():
    # packed bytes (K padded to 128-row blocks) must stay below 2^31
    q4.check_shape(65536, 65536 - 8, 128)
    with pytest.raises(NotImplementedError, match="2\\^31"):
        q4.check_shape(65536, 65536 + 8, 128)


def test_last_error_is_thread_local():
    import threading
    lib = q4.load_library()
    assert lib.q4_check_shape(512, 12, 128) == q4.ERR_INVALID_ARG
    seen = {}

    def other():
        seen["status"] = lib.q4_last_status()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["status"] == q4.OK
    assert lib.q4_last_status() == q4.ERR_INVALID_ARG
    assert b"multiple of 8" in lib.q4_last_error()


def test_null_handle_calls_fail_cleanly():
    lib = q4.load_library()
    assert lib.q4_path_for(None, 1) == -1
    assert lib.q4_matmul(None, None, None, 1, None) == q4.ERR_INVALID_ARG
    assert lib.q4_dequant_dump(None, 1, None, None) == q4.ERR_INVALID_ARG
    lib.q4_free(None)


def test_read_probe_rejects_bad_arguments():
    # (each check runs before anything is enqueued, so no GPU is needed; the
    # non-null pointer is never dereferenced)
    lib = q4.load_library()
    sink = ctypes.c_void_p(0x2000)
    assert lib.q4_read_probe(None, 16384, sink, None) == q4.ERR_INVALID_ARG
    assert lib.q4_read_probe(ctypes.c_void_p(0x1000), 16384, None, None) == q4.ERR_INVALID_ARG
    assert lib.q4_read_probe(ctypes.c_void_p(0x1008), 16384, sink, None) == q4.ERR_INVALID_ARG
    assert b"16-byte aligned" in lib.q4_last_error()
    for bad in (0, 100, 16384 + 16):
        assert lib.q4_read_probe(ctypes.c_void_p(0x1000), bad, sink, None) == q4.ERR_INVALID_ARG
        assert b"multiple of 16384" in lib.q4_last_error()
