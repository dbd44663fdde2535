"""Pins for the CPU oracle: each test checks it against something other than
itself -- a library routine, exact rational brute force, a closed form or an
invariant the pages state -- so that a dropped term, a wrong sign or index, or
a transposed operand in the oracle fails at least one of them.

Passages:
 - "GPTQ's 'Exllama Kernel Not Installed' Warning", "Why the kernel is
   missing": 32-bit words carrying 4-bit codes, one scale and zero per group.
 - same page, "What the fallback actually does": fused route and fallback
   route must give identical products.
 - "Implementation: Predibase Lorax GPTQ Exllama V1", Description and I/O
   contract: g_idx None or trivial means no act-order.
 - GPTQModel wiki "Inference Backends", "Runtime cache lifetime": the
   act-order reorder comes from one stable argsort of g_idx.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from tests.packing import pack_cols, pack_rows, pack_word_py

# ---------------------------------------------------------------- binary16 ---

def test_half_to_double_exhaustive(oracle_mod):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)        # library routine
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _finite_halves():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return np.sort(np.unique(v[np.isfinite(v)].astype(np.float64)))


def test_double_to_half_exact_values(oracle_mod):
    vals = _finite_halves()
    got = oracle_mod.double_to_half(vals)
    ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_double_to_half_midpoints_ties_to_even(oracle_mod):
    vals = _finite_halves()
    mids = (vals[:-1] + vals[1:]) / 2.0             # exact in float64
    got = oracle_mod.double_to_half(mids)
    ref = mids.astype(np.float16).view(np.uint16)  # numpy rounds ties to even
    assert np.array_equal(got, ref)
    # and a hand case: 1 + 2^-11 is the midpoint of 1 and 1 + 2^-10 -> 1 (even)
    assert oracle_mod.double_to_half([1.0 + 2.0 ** -11])[0] == 0x3C00
    assert oracle_mod.double_to_half([1.0 + 3 * 2.0 ** -11])[0] == 0x3C02


def test_double_to_half_random_and_edges(oracle_mod):
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 6, 200000),
        np.array([65504.0, 65519.999, 65520.0, 70000.0, -65520.0, 2.0 ** -24,
                  2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 1e-30, -0.0, 0.0,
                  np.inf, -np.inf]),
    ])
    got = oracle_mod.double_to_half(vals)
    ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    nan = oracle_mod.double_to_half([np.nan])[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0


# ---------------------------------------------------------------- unpack ---

def test_hand_words():
    import oracle
    # nibble i of word (0, n) is the code of row k = i, lowest bits first
    qw = np.array([[0x76543210, pack_word_py(range(8, 16))]], dtype=np.int64).astype(np.int32)
    assert qw[0, 1] < 0                         # 0xFEDCBA98 sets the sign bit
    q = oracle.unpack_qweight(qw, 8)
    assert q[:, 0].tolist() == list(range(8))
    assert q[:, 1].tolist() == list(range(8, 16))
    # zeros are packed along N: word (g, c) holds columns 8c..8c+7
    qz = np.array([[0x76543210, pack_word_py(range(8, 16))]], dtype=np.int32)
    z = oracle.unpack_qzeros(qz, 16)
    assert z[0].tolist() == list(range(16))


def test_golden_nibble_fixture(oracle_mod):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "nibble_order.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    for word_hex, codes in rows:
        w = np.array([[np.uint32(int(word_hex, 16))]], dtype=np.uint32).view(np.int32)
        q = oracle_mod.unpack_qweight(w, 8)[:, 0]
        assert "".join("%x" % c for c in q) == codes, word_hex
        z = oracle_mod.unpack_qzeros(w, 8)[0]
        assert "".join("%x" % c for c in z) == codes, word_hex


@pytest.mark.parametrize("K,N", [(8, 8), (64, 24), (512, 512)])
def test_pack_unpack_round_trip(oracle_mod, K, N):
    rng = np.random.default_rng(K * 1000 + N)
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    assert np.array_equal(oracle_mod.unpack_qweight(pack_rows(q), K), q)
    z = rng.integers(0, 16, size=(K // 8, N), dtype=np.uint8)
    assert np.array_equal(oracle_mod.unpack_qzeros(pack_cols(z), N), z)


# ---------------------------------------------------------------- dequant ---

def _codes_layer(rng, K, N, G, scale_bits=None):
    ng = -(-K // G)
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    z = rng.integers(0, 16, size=(ng, N), dtype=np.uint8)
    if scale_bits is None:
        s = rng.uniform(0.005, 0.02, size=(ng, N)).astype(np.float16)
    else:
        s = scale_bits
    return q, z, s


def test_dequant_brute_force_fractions(oracle_mod):
    rng = np.random.default_rng(7)
    K, N, G = 64, 16, 32
    q, z, s = _codes_layer(rng, K, N, G)
    s[0, 0] = np.float16(-0.0107)   # negative scale
    s[1, 3] = np.float16(6.0e-6)    # subnormal scale
    W = oracle_mod.dequant32(pack_rows(q), pack_cols(z), s, None, K, N, G)
    for k in range(K):
        for n in range(N):
            g = k // G
            exact = Fraction(float(s[g, n])) * (int(q[k, n]) - int(z[g, n]))
            assert Fraction(float(W[k, n])) == exact, (k, n)


def test_dequant16_is_rne_of_exact_product(oracle_mod):
    rng = np.random.default_rng(8)
    K, N, G = 256, 64, 32
    q, z, s = _codes_layer(rng, K, N, G)
    dq = oracle_mod.dequant16(pack_rows(q), pack_cols(z), s, None, K, N, G)
    d = q.astype(np.int32) - np.repeat(z.astype(np.int32), G, axis=0)
    exact = np.repeat(s.astype(np.float32), G, axis=0) * d.astype(np.float32)  # exact in fp32
    ref = exact.astype(np.float16).view(np.uint16)                              # library RNE
    assert np.array_equal(dq, ref)


def test_dequant_closed_forms(oracle_mod):
    rng = np.random.default_rng(9)
    K, N, G = 64, 32, 32
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    # q == z in every group -> W == 0 exactly
    zq = np.zeros((K // G, N), dtype=np.uint8)
    qeq = np.repeat(rng.integers(0, 16, size=(K // G, N), dtype=np.uint8), G, axis=0)
    zq[:] = qeq[::G]
    s = rng.uniform(0.005, 0.02, size=(K // G, N)).astype(np.float16)
    W = oracle_mod.dequant32(pack_rows(qeq), pack_cols(zq), s, None, K, N, G)
    assert np.all(W == 0)
    # s == 1, z == 0 -> W == q
    one = np.ones((K // G, N), dtype=np.float16)
    W = oracle_mod.dequant32(pack_rows(q), pack_cols(np.zeros((K // G, N), np.uint8)), one,
                             None, K, N, G)
    assert np.array_equal(W, q.astype(np.float32))
    # s == 2^-j, z == 8 -> W == (q - 8) * 2^-j, exact in fp16 as well
    for j in (0, 3, 10):
        sj = np.full((K // G, N), 2.0 ** -j, dtype=np.float16)
        z8 = np.full((K // G, N), 8, dtype=np.uint8)
        dq = oracle_mod.dequant16(pack_rows(q), pack_cols(z8), sj, None, K, N, G)
        ref = ((q.astype(np.float64) - 8) * 2.0 ** -j).astype(np.float16).view(np.uint16)
        assert np.array_equal(dq, ref)


def test_group_indexing_uses_k_over_g(oracle_mod):
    """Scale of group g multiplies rows g*G .. g*G+G-1 only (wrong index or a
    transposed scale table fails this)."""
    K, N, G = 96, 8, 32
    q = np.full((K, N), 9, dtype=np.uint8)
    z = np.full((3, N), 8, dtype=np.uint8)
    s = np.array([[1.0] * N, [2.0] * N, [4.0] * N], dtype=np.float16)
    s[2, 5] = 0.5
    W = oracle_mod.dequant32(pack_rows(q), pack_cols(z), s, None, K, N, G)
    assert np.all(W[:32] == 1) and np.all(W[32:64] == 2)
    assert np.all(W[64:, 5] == 0.5) and np.all(W[64:, :5] == 4)
    # ragged last group: K = 96, G = 64 -> 2 groups, the second has 32 rows
    s2 = np.array([[1.0] * N, [3.0] * N], dtype=np.float16)
    W = oracle_mod.dequant32(pack_rows(q), pack_cols(z[:2]), s2, None, K, N, 64)
    assert np.all(W[:64] == 1) and np.all(W[64:] == 3)


# ---------------------------------------------------------------- matmul ---

def _exact_product(x16, q, z, s, G, g_idx=None, bias=None):
    """Exact rational y = x @ W (+ bias) with Python integers.
    x (fp16) is a multiple of 2^-24; W = s*(q-z) is a multiple of 2^-24 too
    (any fp16 scale is), so every product is an integer times 2^-48."""
    M, K = x16.shape
    N = q.shape[1]
    X = [[int(Fraction(float(v)) * (1 << 24)) for v in row] for row in x16]
    Wi = [[0] * N for _ in range(K)]
    for k in range(K):
        g = int(g_idx[k]) if g_idx is not None else k // G
        for n in range(N):
            Wi[k][n] = int(Fraction(float(s[g, n])) * (1 << 24)) * (int(q[k, n]) - int(z[g, n]))
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = 0
            for k in range(K):
                acc += X[m][k] * Wi[k][n]
            r = Fraction(acc, 1 << 48)
            if bias is not None:
                r += Fraction(float(bias[n]))
            row.append(r)
        out.append(row)
    return out


def test_matmul_exact_brute_force_small(oracle_mod):
    rng = np.random.default_rng(11)
    M, K, N, G = 3, 96, 16, 32
    q, z, s = _codes_layer(rng, K, N, G)
    x = rng.standard_normal((M, K)).astype(np.float16)
    b = rng.normal(0, 0.1, size=N).astype(np.float16)
    y, A = oracle_mod.matmul(x, pack_rows(q), pack_cols(z), s, None, K, N, G, bias=b)
    ex = _exact_product(x, q, z, s, G, bias=b)
    for m in range(M):
        for n in range(N):
            # s >= 2^-8 makes W a multiple of 2^-18 and x is a multiple of
            # 2^-24, so every partial sum is a multiple of 2^-42 below 2^8:
            # exact in double
            assert Fraction(y[m, n]) == ex[m][n], (m, n)


def test_matmul_exact_brute_force_tiny_workload(oracle_mod):
    """The 512x512 G=128 layer: with |x| < 8 and |W| <= 0.3 every partial sum
    is a multiple of 2^-42 below 2^11, so the double sum is exact."""
    L = synth.make_layer(512, 512, 128, 1, seed=synth.layer_seed("tiny", 0))
    import oracle
    q = oracle.unpack_qweight(L.qweight, 512)
    z = oracle.unpack_qzeros(L.qzeros, 512)
    # cross-check the unpack against the independent packer first
    assert np.array_equal(pack_rows(q), L.qweight)
    assert np.array_equal(pack_cols(z), L.qzeros)
    assert np.max(np.abs(L.x.astype(np.float64))) < 8
    y, _ = oracle_mod.matmul(L.x, L.qweight, L.qzeros, L.scales, None, 512, 512, 128)
    X = (L.x.astype(np.float64) * 2.0 ** 24).astype(np.int64)          # exact
    S = (np.repeat(L.scales, 128, axis=0).astype(np.float64) * 2.0 ** 18).astype(np.int64)
    assert np.array_equal(S.astype(np.float64) * 2.0 ** -18,
                          np.repeat(L.scales, 128, axis=0).astype(np.float64))  # s >= 2^-8
    Wi = S * (q.astype(np.int64) - np.repeat(z.astype(np.int64), 128, axis=0))
    # integer matmul in Python ints column by column (no overflow possible)
    ref = [sum(int(a) * int(b) for a, b in zip(X[0], Wi[:, n])) for n in range(512)]
    got = [Fraction(v) * (1 << 42) for v in y[0]]
    assert got == [Fraction(r) for r in ref]


def test_matmul_special_case_numpy(oracle_mod):
    """s = 1, z = 0: W is the integer code matrix and y = x @ q exactly, which
    numpy's float64 matmul also gives exactly for these magnitudes."""
    rng = np.random.default_rng(12)
    M, K, N, G = 4, 256, 40, 64
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    z = np.zeros((K // G, N), dtype=np.uint8)
    s = np.ones((K // G, N), dtype=np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    y, A = oracle_mod.matmul(x, pack_rows(q), pack_cols(z), s, None, K, N, G)
    ref = x.astype(np.float64) @ q.astype(np.float64)
    assert np.array_equal(y, ref)
    assert np.array_equal(A, np.abs(x.astype(np.float64)) @ q.astype(np.float64))


def test_fused_equals_fallback_bitwise(oracle_mod):
    L = synth.make_layer(1024, 264, 128, 5, seed=3, act_order=True, bias=True)
    a, _ = oracle_mod.matmul(L.x, L.qweight, L.qzeros, L.scales, L.g_idx, L.K, L.N, L.G,
                             bias=L.bias, route="fused")
    b, _ = oracle_mod.matmul(L.x, L.qweight, L.qzeros, L.scales, L.g_idx, L.K, L.N, L.G,
                             bias=L.bias, route="fallback")
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


def test_matmul_at_matches_full(oracle_mod):
    L = synth.make_layer(512, 136, 32, 6, seed=4, bias=True)
    y, A = oracle_mod.matmul(L.x, L.qweight, L.qzeros, L.scales, None, L.K, L.N, L.G,
                             bias=L.bias)
    rng = np.random.default_rng(0)
    ms = rng.integers(0, 6, 50)
    ns = rng.integers(0, 136, 50)
    ys, As = oracle_mod.matmul_at(L.x, L.qweight, L.qzeros, L.scales, None, L.K, L.N, L.G,
                                  ms, ns, bias=L.bias)
    assert np.array_equal(ys, y[ms, ns]) and np.array_equal(As, A[ms, ns])


def test_trivial_g_idx_equals_none(oracle_mod):
    L = synth.make_layer(512, 64, 128, 2, seed=5)
    g = (np.arange(512) // 128).astype(np.int32)
    a, _ = oracle_mod.matmul(L.x, L.qweight, L.qzeros, L.scales, None, 512, 64, 128)
    b, _ = oracle_mod.matmul(L.x, L.qweight, L.qzeros, L.scales, g, 512, 64, 128)
    assert np.array_equal(a, b)


def _physically_permuted(oracle_mod, L):
    perm = np.argsort(L.g_idx, kind="stable")            # library stable argsort
    assert np.array_equal(L.g_idx[perm], np.arange(L.K) // L.G)
    q = oracle_mod.unpack_qweight(L.qweight, L.K)
    return perm, pack_rows(q[perm]), L.x[:, perm]


def test_act_order_equals_physical_permutation_exact(oracle_mod):
    """Non-trivial g_idx == trivial g_idx on K-permuted weights and activations.
    Small K: both double sums are exact, so the results are bit-identical."""
    L = synth.make_layer(256, 48, 32, 3, seed=6, act_order=True)
    perm, qw_p, x_p = _physically_permuted(oracle_mod, L)
    a, _ = oracle_mod.matmul(L.x, L.qweight, L.qzeros, L.scales, L.g_idx, L.K, L.N, L.G)
    b, _ = oracle_mod.matmul(x_p, qw_p, L.qzeros, L.scales, None, L.K, L.N, L.G)
    assert np.array_equal(a, b)


def test_act_order_equals_physical_permutation_large(oracle_mod):
    """Same invariant at K = 4096: two summation orders, |diff| <= 2 K 2^-53 A."""
    L = synth.make_layer(4096, 64, 128, 2, seed=7, act_order=True)
    perm, qw_p, x_p = _physically_permuted(oracle_mod, L)
    a, A = oracle_mod.matmul(L.x, L.qweight, L.qzeros, L.scales, L.g_idx, L.K, L.N, L.G)
    b, _ = oracle_mod.matmul(x_p, qw_p, L.qzeros, L.scales, None, L.K, L.N, L.G)
    assert np.all(np.abs(a - b) <= 2 * L.K * 2.0 ** -53 * A)
    assert not np.array_equal(L.g_idx, np.arange(L.K) // L.G)


def test_act_order_wrong_permutation_is_detected(oracle_mod):
    """The invariant has teeth: permuting x with a different permutation moves
    the result far outside the bound."""
    L = synth.make_layer(256, 16, 32, 1, seed=8, act_order=True)
    perm, qw_p, x_p = _physically_permuted(oracle_mod, L)
    a, A = oracle_mod.matmul(L.x, L.qweight, L.qzeros, L.scales, L.g_idx, L.K, L.N, L.G)
    b, _ = oracle_mod.matmul(L.x[:, np.argsort(perm)], qw_p, L.qzeros, L.scales, None,
                             L.K, L.N, L.G)
    assert not np.all(np.abs(a - b) <= 1e-3 * A)


def test_group_replication_invariant(oracle_mod):
    """G=128 with each group's (s, z) copied into four G=32 groups gives the
    identical W, hence the identical y."""
    L = synth.make_layer(512, 64, 128, 2, seed=9)
    z = oracle_mod.unpack_qzeros(L.qzeros, 64)
    z4 = np.repeat(z, 4, axis=0)
    s4 = np.repeat(L.scales, 4, axis=0)
    a, _ = oracle_mod.matmul(L.x, L.qweight, L.qzeros, L.scales, None, 512, 64, 128)
    b, _ = oracle_mod.matmul(L.x, L.qweight, pack_cols(z4), s4, None, 512, 64, 32)
    assert np.array_equal(a, b)


def test_bias_adds_exactly(oracle_mod):
    L = synth.make_layer(512, 64, 128, 2, seed=10, bias=True)
    a, _ = oracle_mod.matmul(L.x, L.qweight, L.qzeros, L.scales, None, 512, 64, 128)
    b, _ = oracle_mod.matmul(L.x, L.qweight, L.qzeros, L.scales, None, 512, 64, 128,
                             bias=L.bias)
    # all partial sums are exact here (see the tiny-workload pin), so the
    # difference is the bias itself, exactly
    assert np.array_equal(b - a, np.broadcast_to(L.bias.astype(np.float64), a.shape))


def test_degenerate_and_error_cases(oracle_mod):
    L = synth.make_layer(64, 16, 32, 0, seed=11)
    y, A = oracle_mod.matmul(L.x, L.qweight, L.qzeros, L.scales, None, 64, 16, 32)
    assert y.shape == (0, 16)
    # groupsize <= 0: one group over all of K
    L1 = synth.make_layer(64, 16, -1, 2, seed=12)
    assert L1.scales.shape == (1, 16)
    y1, _ = oracle_mod.matmul(L1.x, L1.qweight, L1.qzeros, L1.scales, None, 64, 16, -1)
    y2, _ = oracle_mod.matmul(L1.x, L1.qweight, L1.qzeros, L1.scales, None, 64, 16, 64)
    assert np.array_equal(y1, y2)
    with pytest.raises(oracle_mod.OracleError):
        bad = np.full(64, 2, dtype=np.int32)   # only groups 0, 1 exist
        oracle_mod.matmul(L.x, L.qweight, L.qzeros, L.scales, bad, 64, 16, 32)
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.dequant32(L.qweight, L.qzeros, L.scales, None, 60, 16, 32)


def test_tolerance_scale_is_sum_abs(oracle_mod):
    """A = sum_k |x W|: with all-positive x and W it equals y itself."""
    K, N, G = 64, 8, 32
    q = np.full((K, N), 12, dtype=np.uint8)
    z = np.full((2, N), 4, dtype=np.uint8)
    s = np.full((2, N), 0.25, dtype=np.float16)
    x = np.full((1, K), 0.5, dtype=np.float16)
    y, A = oracle_mod.matmul(x, pack_rows(q), pack_cols(z), s, None, K, N, G)
    assert np.all(y == K * 0.5 * 2.0) and np.array_equal(A, y)
    y2, A2 = oracle_mod.matmul(-x, pack_rows(q), pack_cols(z), s, None, K, N, G)
    assert np.array_equal(y2, -y) and np.array_equal(A2, A)


def test_concatenated_layers_equal_their_parts(oracle_mod):
    """Projection fusion is a column concatenation: the oracle on the stacked
    layers equals the parts' results side by side, bit for bit (every column
    is computed independently), including the packed zeros of parts whose
    widths are not multiples of 64 and a part without bias."""
    K, G = 256, 64
    parts = [synth.make_layer(K, n, G, 3, seed=s, bias=b)
             for n, s, b in ((40, 1, True), (16, 2, False), (72, 3, True))]
    x = parts[0].x
    cat = synth.concat_layers(parts, x)
    assert cat.N == 128 and cat.qzeros.shape == (K // G, 16)
    y, A = oracle_mod.matmul(x, cat.qweight, cat.qzeros, cat.scales, None, K, cat.N, G, bias=cat.bias)
    outs = [oracle_mod.matmul(x, p.qweight, p.qzeros, p.scales, None, K, p.N, G, bias=p.bias)
            for p in parts]
    assert np.array_equal(y, np.hstack([o[0] for o in outs]))
    assert np.array_equal(A, np.hstack([o[1] for o in outs]))
    dq = oracle_mod.dequant16(cat.qweight, cat.qzeros, cat.scales, None, K, cat.N, G)
    assert np.array_equal(dq, np.hstack([oracle_mod.dequant16(p.qweight, p.qzeros, p.scales, None,
                                                              K, p.N, G) for p in parts]))
    with pytest.raises(ValueError):
        synth.concat_layers([parts[0], synth.make_layer(128, 16, G, 3, seed=4)])


def test_missing_zeros_mean_symmetric_eight(oracle_mod):
    """qzeros absent (a symmetric layer): the zero point is 2^(bits-1) = 8
    ("Inference Backends", packing-control row "Missing zeros"). Pinned two
    ways: equal to explicit zero words 0x88888888, and the closed form
    W = s * (q - 8) on hand-built codes."""
    L = synth.make_layer(256, 40, 64, 2, seed=11)
    eights = np.full_like(L.qzeros, np.int32(np.uint32(0x88888888).view(np.int32)))
    a = oracle_mod.matmul(L.x, L.qweight, None, L.scales, None, 256, 40, 64)
    b = oracle_mod.matmul(L.x, L.qweight, eights, L.scales, None, 256, 40, 64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(oracle_mod.dequant16(L.qweight, None, L.scales, None, 256, 40, 64),
                          oracle_mod.dequant16(L.qweight, eights, L.scales, None, 256, 40, 64))
    K, N, G = 16, 8, 16
    q = np.arange(K * N, dtype=np.int64).reshape(K, N) % 16
    W = oracle_mod.dequant32(pack_rows(q), None, np.ones((1, N), np.float16), None, K, N, G)
    assert np.array_equal(W, (q - 8).astype(np.float32))


# ---------------------------------------------------------------- bfloat16 ---
# Activation format: GPTQModel wiki "Inference Backends", hardware table
# (ExLlama v2 row): the activation dtype (FP16, BF16 or FP32) is kept, with
# FP16 scales and FP32 accumulation. bfloat16 is the upper half of a binary32
# word, so numpy's float32 decoding and torch's float32 -> bfloat16 rounding
# are independent references for the oracle's own conversions.

def _torch_bf16_bits(v32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_decode_exhaustive(oracle_mod):
    bits = np.arange(1 << 16, dtype=np.uint32)
    ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = oracle_mod.bf16_to_double(bits.astype(np.uint16))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # closed forms
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x0080: 2.0 ** -126,
             0x0001: 2.0 ** -133, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127}
    for b, v in cases.items():
        assert oracle_mod.bf16_to_double(np.array([b], dtype=np.uint16))[0] == v, hex(b)


def test_double_to_bf16_matches_torch(oracle_mod):
    rng = np.random.default_rng(21)
    pats = rng.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32)
    pats[:20000] = (pats[:20000] & 0xFFFF0000) | 0x8000        # exact ties
    pats[20000:30000] &= 0x807FFFFF                             # bfloat16 subnormal range
    v = pats.view(np.float32)
    keep = np.isfinite(v)
    v = v[keep]
    got = oracle_mod.double_to_bf16(v.astype(np.float64))
    ref = _torch_bf16_bits(v)
    assert np.array_equal(got, ref)


def test_double_to_bf16_hand_cases(oracle_mod):
    d = oracle_mod.double_to_bf16
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to the even fraction
    assert d([1 + 2.0 ** -8])[0] == 0x3F80
    assert d([1 + 3 * 2.0 ** -8])[0] == 0x3F82
    assert d([1 + 2.0 ** -8 + 2.0 ** -30])[0] == 0x3F81
    assert d([-(1 + 2.0 ** -8)])[0] == 0xBF80
    assert d([(2 - 2.0 ** -8) * 2.0 ** 127])[0] == 0x7F80     # halfway to 2^128: overflow
    assert d([(2 - 2.0 ** -7) * 2.0 ** 127])[0] == 0x7F7F
    assert d([2.0 ** -134])[0] == 0x0000                      # half the smallest subnormal
    assert d([3 * 2.0 ** -134])[0] == 0x0002
    assert d([70000.0])[0] == 0x4789                          # beyond binary16's range


def test_dequant_bf16_is_one_rounding(oracle_mod):
    L = synth.make_layer(256, 64, 32, 1, seed=synth.layer_seed("bf16 pin", 1))
    W = oracle_mod.dequant32(L.qweight, L.qzeros, L.scales, None, 256, 64, 32)
    got = oracle_mod.dequant_bf16(L.qweight, L.qzeros, L.scales, None, 256, 64, 32)
    assert np.array_equal(got, _torch_bf16_bits(W))
    # the rounding matters: truncating the fp32 word differs somewhere
    assert not np.array_equal(got, (W.view(np.uint32) >> 16).astype(np.uint16))


def test_bf16_route_equals_f16_route_on_shared_values(oracle_mod):
    """Activations with at most 8 significant bits inside binary16's normal
    range are exact in both formats: the two formats then give the same y."""
    rng = np.random.default_rng(22)
    M, K, N, G = 3, 256, 48, 64
    L = synth.make_layer(K, N, G, M, seed=synth.layer_seed("bf16 pin", 2), act_order=True)
    xv = rng.integers(-255, 256, size=(M, K)).astype(np.float64) * 2.0 ** -6
    bv = rng.integers(-255, 256, size=N).astype(np.float64) * 2.0 ** -9
    x16, b16 = xv.astype(np.float16), bv.astype(np.float16)
    xb = (xv.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bb = (bv.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle_mod.bf16_to_double(xb), xv)
    y16, A16 = oracle_mod.matmul(x16, L.qweight, L.qzeros, L.scales, L.g_idx, K, N, G, bias=b16)
    yb, Ab = oracle_mod.matmul(xb, L.qweight, L.qzeros, L.scales, L.g_idx, K, N, G, bias=bb,
                               xfmt="bf16")
    assert np.array_equal(y16, yb) and np.array_equal(A16, Ab)
    yf, _ = oracle_mod.matmul(xb, L.qweight, L.qzeros, L.scales, L.g_idx, K, N, G, bias=bb,
                              xfmt="bf16", route="fallback")
    assert np.array_equal(yf, yb)
    ms, ns = np.array([0, 2, 1]), np.array([5, 47, 0])
    ya, _ = oracle_mod.matmul_at(xb, L.qweight, L.qzeros, L.scales, L.g_idx, K, N, G, ms, ns,
                                 bias=bb, xfmt="bf16")
    assert np.array_equal(ya, yb[ms, ns])


def test_bf16_activations_beyond_binary16_range(oracle_mod):
    """Single non-zero activations give y = x * W exactly: 2^40 (beyond
    binary16) and 2^-130 (a bfloat16 subnormal); zero activations give the
    bias."""
    K, N, G = 128, 16, 32
    L = synth.make_layer(K, N, G, 1, seed=synth.layer_seed("bf16 pin", 3))
    W = oracle_mod.dequant32(L.qweight, L.qzeros, L.scales, None, K, N, G).astype(np.float64)
    x = np.zeros((3, K), dtype=np.uint16)
    x[0, 7] = 0x5380                  # 2^40
    x[1, 99] = 0x0008                 # 8 * 2^-133 = 2^-130
    bias = np.arange(N, dtype=np.uint16) + 0x3F80        # 1, 1 + 2^-7, ...
    y, _ = oracle_mod.matmul(x, L.qweight, L.qzeros, L.scales, None, K, N, G, xfmt="bf16")
    assert np.array_equal(y[0], 2.0 ** 40 * W[7]) and np.array_equal(y[1], 2.0 ** -130 * W[99])
    assert not y[2].any()
    yb, _ = oracle_mod.matmul(x, L.qweight, L.qzeros, L.scales, None, K, N, G, bias=bias,
                              xfmt="bf16")
    assert np.array_equal(yb[2], 1 + np.arange(N) * 2.0 ** -7)
    with pytest.raises(ValueError):
        oracle_mod.matmul(x, L.qweight, L.qzeros, L.scales, None, K, N, G, xfmt="f32")


# ---------------------------------------------------------------- 8-bit -----
# GPTQModel wiki "Inference Backends": GPTQ kernels declare 4- and 8-bit
# weights (backend catalogue); the native 8-bit path keeps the checkpoint's
# qweight, qzeros, scales and g_idx ("Runtime cache lifetime"). Reading: four
# 8-bit codes a word, packed as the 4-bit ones (code i in bits 8i..8i+7,
# qweight along K, qzeros along N); symmetric zero point 2^(8-1) = 128.

def test_hand_words_8bit(oracle_mod):
    qw = np.array([[0x04030201, np.uint32(0xFFFEFDFC).view(np.int32)]], dtype=np.int64).astype(np.int32)
    q = oracle_mod.unpack_qweight(qw, 4, bits=8)
    assert q[:, 0].tolist() == [1, 2, 3, 4] and q[:, 1].tolist() == [252, 253, 254, 255]
    qz = np.array([[0x04030201, 0x08070605]], dtype=np.int32)
    assert oracle_mod.unpack_qzeros(qz, 8, bits=8)[0].tolist() == [1, 2, 3, 4, 5, 6, 7, 8]


@pytest.mark.parametrize("K,N", [(8, 8), (64, 24), (512, 136)])
def test_pack_unpack_round_trip_8bit(oracle_mod, K, N):
    rng = np.random.default_rng(K * 7 + N)
    q = rng.integers(0, 256, size=(K, N), dtype=np.uint8)
    assert np.array_equal(oracle_mod.unpack_qweight(pack_rows(q, 8), K, bits=8), q)
    z = rng.integers(0, 256, size=(K // 8, N), dtype=np.uint8)
    assert np.array_equal(oracle_mod.unpack_qzeros(pack_cols(z, 8), N, bits=8), z)


def test_dequant_8bit_brute_force_fractions(oracle_mod):
    rng = np.random.default_rng(17)
    K, N, G = 64, 16, 32
    q = rng.integers(0, 256, size=(K, N), dtype=np.uint8)
    z = rng.integers(0, 256, size=(K // G, N), dtype=np.uint8)
    s = rng.uniform(0.0005, 0.002, size=(K // G, N)).astype(np.float16)
    s[0, 0] = np.float16(-0.00107)
    s[1, 3] = np.float16(6.0e-6)            # subnormal
    W = oracle_mod.dequant32(pack_rows(q, 8), pack_cols(z, 8), s, None, K, N, G, bits=8)
    for k in range(K):
        for n in range(N):
            g = k // G
            exact = Fraction(float(s[g, n])) * (int(q[k, n]) - int(z[g, n]))
            assert Fraction(float(W[k, n])) == exact, (k, n)
    dq = oracle_mod.dequant16(pack_rows(q, 8), pack_cols(z, 8), s, None, K, N, G, bits=8)
    ref = W.astype(np.float16).view(np.uint16)
    assert np.array_equal(dq, ref)
    db = oracle_mod.dequant_bf16(pack_rows(q, 8), pack_cols(z, 8), s, None, K, N, G, bits=8)
    assert np.array_equal(db, _torch_bf16_bits(W))


def test_matmul_8bit_exact_brute_force(oracle_mod):
    rng = np.random.default_rng(18)
    M, K, N, G = 2, 64, 16, 32
    q = rng.integers(0, 256, size=(K, N), dtype=np.uint8)
    z = rng.integers(0, 256, size=(K // G, N), dtype=np.uint8)
    s = rng.uniform(0.0005, 0.002, size=(K // G, N)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    b = rng.normal(0, 0.1, size=N).astype(np.float16)
    y, _ = oracle_mod.matmul(x, pack_rows(q, 8), pack_cols(z, 8), s, None, K, N, G, bias=b, bits=8)
    ex = _exact_product(x, q, z, s, G, bias=b)
    for m in range(M):
        for n in range(N):
            # every product is exact in double, the 64-term sum may round
            # (up to ~55 significant bits): 64 * 2^-53 relative at most, far
            # below any wrong code, zero or index (at least min|s x| ~ 1e-7)
            assert abs(Fraction(y[m, n]) - ex[m][n]) <= Fraction(1, 1 << 40) * (1 + abs(ex[m][n])), (m, n)


def test_8bit_equals_4bit_on_small_codes(oracle_mod):
    """Codes and zeros below 16 packed as 8-bit words give exactly the 4-bit
    layer's results (two different unpackers, the same layer)."""
    rng = np.random.default_rng(19)
    M, K, N, G = 3, 256, 40, 64
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    z = rng.integers(0, 16, size=(K // G, N), dtype=np.uint8)
    s = rng.uniform(0.005, 0.02, size=(K // G, N)).astype(np.float16)
    x = rng.standard_normal((M, K)).astype(np.float16)
    gi = synth.make_layer(K, N, G, 1, seed=3, act_order=True).g_idx
    y4, A4 = oracle_mod.matmul(x, pack_rows(q), pack_cols(z), s, gi, K, N, G)
    y8, A8 = oracle_mod.matmul(x, pack_rows(q, 8), pack_cols(z, 8), s, gi, K, N, G, bits=8)
    assert np.array_equal(y4, y8) and np.array_equal(A4, A8)
    y8f, _ = oracle_mod.matmul(x, pack_rows(q, 8), pack_cols(z, 8), s, gi, K, N, G, bits=8,
                               route="fallback")
    assert np.array_equal(y8f, y8)
    ms, ns = np.array([0, 2, 1]), np.array([0, 39, 7])
    ya, _ = oracle_mod.matmul_at(x, pack_rows(q, 8), pack_cols(z, 8), s, gi, K, N, G, ms, ns, bits=8)
    assert np.array_equal(ya, y8[ms, ns])


def test_8bit_missing_zeros_mean_128(oracle_mod):
    K, N, G = 16, 8, 16
    q = (np.arange(K * N, dtype=np.int64).reshape(K, N) * 37) % 256
    W = oracle_mod.dequant32(pack_rows(q, 8), None, np.ones((1, N), np.float16), None, K, N, G, bits=8)
    assert np.array_equal(W, (q - 128).astype(np.float32))
    with pytest.raises(ValueError):
        oracle_mod.dequant32(pack_rows(q, 8), None, np.ones((1, N), np.float16), None, K, N, G, bits=6)
