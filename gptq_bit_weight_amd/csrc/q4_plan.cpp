// Host-side argument checks, act-order planning and launch planning for
// libq4. Nothing in this file calls the HIP runtime, so every function here
// can be exercised on a machine without a GPU.
#include "q4_internal.h"

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <numeric>
#include <vector>

namespace q4 {

static thread_local q4_status t_status = Q4_OK;
static thread_local char t_message[512] = "";

q4_status fail(q4_status st, const char* fmt, ...)
{
    t_status = st;
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(t_message, sizeof(t_message), fmt, ap);
    va_end(ap);
    return st;
}

q4_status last_status() { return t_status; }
const char* last_message() { return t_message; }

// Shape rules of the GPU path. The checkpoint format only needs K % 8 and
// N % 8 (whole packed words along K for qweight and along N for qzeros); the
// kernels also walk K in steps of 32 (one MFMA k-block), hence K % 32.
q4_status check_shape(int K, int N, int groupsize, int* G_out, int bits)
{
    if (K <= 0 || N <= 0)
        return fail(Q4_ERR_INVALID_ARG, "K and N must be positive (got K=%d, N=%d)", K, N);
    if (K % 8)
        return fail(Q4_ERR_INVALID_ARG, "K=%d is not a multiple of 8 (qweight packs 8 rows per word)", K);
    if (N % 8)
        return fail(Q4_ERR_INVALID_ARG, "N=%d is not a multiple of 8 (qzeros packs 8 columns per word)", N);
    int G = groupsize;
    if (G == -1)
        G = K;
    else if (G != 32 && G != 64 && G != 128 && G != 256)
        return fail(Q4_ERR_UNSUPPORTED, "groupsize=%d is not one of 32, 64, 128, 256 or -1", groupsize);
    if (K % 32)
        return fail(Q4_ERR_UNSUPPORTED, "K=%d is not a multiple of 32 (the kernels' k-block)", K);
    if (K % G)
        return fail(Q4_ERR_UNSUPPORTED, "K=%d is not a multiple of groupsize=%d", K, G);
    // Byte offsets inside the packed weights (K padded to whole 128-row
    // blocks) stay below 2^31: the kernels mark out-of-range lanes by setting
    // bit 31 of the offset.
    if (bits != 4 && bits != 8) return fail(Q4_ERR_UNSUPPORTED, "bits=%d is not 4 or 8", bits);
    const long long packed = (long long)num_kblocks(K) * (kBlockK * bits / 8) * (long long)N;
    if (packed > (1LL << 31) - 1)
        return fail(Q4_ERR_UNSUPPORTED, "%lld bytes of packed weights exceed 2^31 - 1", packed);
    if (G_out) *G_out = G;
    return Q4_OK;
}

// Stable argsort of g_idx; trivial when g_idx[k] == k / G everywhere.
q4_status plan_actorder(const int32_t* g_idx, int K, int G, int32_t* perm, int* trivial)
{
    const int ng = K / G;
    bool triv = true;
    for (int k = 0; k < K; ++k) {
        if (g_idx[k] < 0 || g_idx[k] >= ng)
            return fail(Q4_ERR_INVALID_ARG, "g_idx[%d]=%d is outside [0, %d)", k, g_idx[k], ng);
        if (g_idx[k] != k / G) triv = false;
    }
    std::vector<int32_t> p(K);
    std::iota(p.begin(), p.end(), 0);
    std::stable_sort(p.begin(), p.end(), [&](int32_t a, int32_t b) { return g_idx[a] < g_idx[b]; });
    for (int k = 0; k < K; ++k)
        if (g_idx[p[k]] != k / G)
            return fail(Q4_ERR_UNSUPPORTED,
                        "act-order groups are not uniform: sorted g_idx[%d]=%d, expected %d "
                        "(every group must hold exactly groupsize=%d rows)",
                        k, g_idx[p[k]], k / G, G);
    std::copy(p.begin(), p.end(), perm);
    *trivial = triv ? 1 : 0;
    return Q4_OK;
}

// Launch plan of the skinny kernel. A workgroup covers 16 * col_tiles
// columns and a contiguous range of 128-row k-blocks that its waves divide.
//  * col_tiles: each 16-column tile is one workgroup's share of the chip, so
//    the tiles should fill whole rounds of CUs: balance(ct) = tiles /
//    (CUs x rounds). Wider tiles reuse each activation fragment across more
//    columns, which pays more the more rows M has (the activation loads grow
//    with M); gain(ct, M) below is that benefit as measured on MI355X over
//    the Llama-7B/70B layer shapes. The plan takes the widest tile with the
//    best balance x gain. For M > 4 the balance counts the K splits that
//    tile width would get while every wave keeps at least 4 k-blocks: a
//    narrow layer then takes wide tiles split in K rather than narrow ones
//    unsplit (M = 16: 28672x8192 35.1 -> 27.9 us with 4 tiles x 2 splits,
//    11008x4096 14.1 -> 11.2 us with 2 x 2). For M <= 4 the partial round
//    trip of a split costs more than the reuse gains (28672x8192, M = 1:
//    2 tiles unsplit 21.4 us, 4 tiles x 2 splits 23.4 us), and with fewer
//    blocks per wave it costs more than the balance gains (4096x4096, M = 8:
//    5.0 us unsplit, 6.5 us with 2 x 2).
//  * splits: K ranges across workgroups, only when the column tiles alone
//    cannot give every CU a workgroup, and only while every wave of every
//    split keeps a k-block. Each split adds a round of fp32 partials and a
//    last-arriver reduction to the critical path.
void plan_gemv(int M, int K, int N, int G, int num_cu, int* col_tiles, int* splits, int bits)
{
    if (num_cu <= 0) num_cu = 256;
    // gain x 100 for 1, 2, 4 tiles: M <= 2, M <= 4, M <= 8, M <= 16,
    // M <= 32. (At M = 1 a wider tile saves little: 8192x28672 ran 21.2 us
    // with one tile a wave against 21.8 us with four, 28672x8192 20.5 us
    // with two against 21.1 us with one, the tiles then filling one round of
    // CUs exactly.) Past 16 rows every activation load serves one k-step of
    // one 16-row block, so wide tiles pay most.
    static const int gain[5][3] = {{100, 104, 104}, {100, 110, 120}, {100, 140, 150}, {100, 160, 190},
                                   {100, 180, 230}};
    const int mi = M <= 2 ? 0 : M <= 4 ? 1 : M <= 8 ? 2 : M <= 16 ? 3 : 4;
    // (groups of 32 rows carry four scale/zero sets per block, and 8-bit
    // blocks are twice the words; four tiles of either do not fit the
    // register file)
    const int max_ct = (G == 32 || bits == 8) ? 2 : kMaxColTiles;
    const int kb = num_kblocks(K);
    // K splits for `tiles` column tiles keeping >= min_blocks k-blocks a wave
    auto splits_for = [&](long long tiles, int min_blocks) {
        int s = 1;
        while (2 * s <= kMaxSplits && tiles * 2 * s <= num_cu && kb >= 2 * s * kGemvWaves * min_blocks) s *= 2;
        return s;
    };
    // At M <= 2 the wider tiles' small gain holds only where one-tile tiles
    // fill whole rounds of CUs; otherwise the finer grid balances the last
    // round better, and one tile wins ties (4096 x 22016 at M = 1: 9.9 us at
    // one tile a wave, 10.4 at two; 28672 x 8192, whose 512 one-tile tiles
    // fill two rounds: 20.7 at two, 21.0 at one).
    const bool fine = mi == 0 && ((N + 15) / 16) % num_cu != 0;
    int ct = 1;
    long long best = -1;
    for (int c = 1, ci = 0; c <= max_ct; c *= 2, ++ci) {
        const long long tiles = (N + 16 * c - 1) / (16 * c);
        const long long rounds = (tiles + num_cu - 1) / num_cu;
        const long long s = M > 4 ? splits_for(tiles, 4) : 1;
        const long long score = tiles * s * 1000 * (fine ? 100 : gain[mi][ci]) / (rounds * num_cu);
        if (score > best || (score == best && !fine)) {
            best = score;
            ct = c;
        }
    }
    const int tiles = (N + 16 * ct - 1) / (16 * ct);
    *col_tiles = ct;
    *splits = splits_for(tiles, 1);
}

// Automatic dispatch between the skinny kernel and the GEMM: the skinny
// kernel for every M it takes. Past 16 rows the GEMM's 64-row tiles are
// bound by their serial k-loop (about 20 us on the 7B MLP shapes for any M
// up to 64), while the skinny kernel with two row blocks measured (M = 17 /
// 24 / 32, us, skinny against GEMM): 4096x11008 11.4 / 12.4 / 13.7 against
// 19.4 / 19.5 / 19.6; 11008x4096 13.0 / 14.9 / 16.6 against 20.2;
// 4096x4096 7.7 / 8.9 / 10.3 against 17.7; 8192x28672 33.1 / 37.6 / 43.3
// against 44.1 / 44.8 / 45.7; 28672x8192 30.9 / 34.6 / 39.7 against
// 44.1 / 45.3 / 46.3.
bool gemv_serves(int M, int K, int N, int G, int bits)
{
    (void)K; (void)N; (void)G; (void)bits;
    return M >= 1 && M <= kGemvMaxM;
}

bool gemv_gathers_x(int M, int K, int splits)
{
    const long long rows = (long long)num_kblocks(K) * kBlockK;
    return splits == 1 && M >= 1 && M <= kGemvXMaxM && rows <= kGemvXRows &&
           (long long)M * (rows + kGemvXPad) <= kGemvXLdsHalfs;
}

// Streaming-GEMM schedule. Two 256-row workgroups share a CU (64 KiB of LDS
// and about 240 VGPRs each), and a CU that holds only one runs a tile at
// about 0.7 times the rate of two (one wave per SIMD leaves the matrix pipe
// idle while that wave dequantizes). With one workgroup per output tile,
// tile counts that are not whole rounds of 2 x CUs leave CUs idle or
// half-used (256 tiles: every CU at one; 688: a third round on a third of
// the chip). Stream-K gives every workgroup the same number of (tile,
// k-tile) iterations instead, at the price of fp32 partials for the tiles
// that straddle two workgroups (measured: 11-13 us a launch at 2048 rows)
// and of more, shorter segments. It is planned below 1.5 rounds of tiles,
// when one-per-tile would also waste more than a tenth of the rounds (256
// tiles: 735 -> 970 TFLOP/s; 688: 869 -> 913); from 1.5 rounds on, the lone
// workgroups of a last half round run fast enough that stream-K measured no
// better (768 tiles: equal; 1792: 1.5% slower).
// The tile width (gemm_waves): 256-column tiles, eight waves a workgroup
// and one workgroup per CU, copy each activation stage once for twice the
// columns and keep two stages in flight (three in 96 KiB of LDS) instead of
// one. Fewer tiles than CUs are shared by stream-K with 256 KiB partial
// sums, which pays when the parts stay long. So the wide tiles serve
// 256-row tiles when there is one for every CU, or one for every two CUs
// with at least 64 k-steps a CU, or any count with at least 128 k-steps a
// CU. Measured (us, planned four-wave against planned eight-wave launches,
// weights from HBM): 4096x11008 at M = 1536 185.7 -> 128.6 (258 wide
// tiles), 2048 172.5 -> 161.9, 4096 334.1 -> 310.4; 11008x4096 at 2048
// (128 tiles, 86 k-steps a CU) 169.8 -> 162.7 but at 1024 (64 tiles)
// 95.9 -> 106.5; 4096x4096 at 2048 (128 tiles, 32 k-steps a CU) 73.4 ->
// 74.9, at 1536 62.5 -> 80.2, at 4096 122.4 -> 113.8; the 70B MLP layers
// 3-12% faster at every M from 768 to 4096 (28672x8192 at 768: 96 tiles,
// 168 k-steps a CU, 348.0 -> 312.1). Left on the table: 4096x11008 at
// M = 768 and 1024 (129 and 172 tiles, 32 and 43 k-steps a CU), 4-6%
// faster wide. 8-bit weights (twice the weight stream) keep the narrow
// tiles: 11008x4096 at M = 2048 1062 TFLOP/s narrow, 993 wide.
int gemm_waves(int M, int N, int K, int num_cu, int bits)
{
    if (num_cu <= 0) num_cu = 256;
    if (gemm_bm(M) < kGemmBM || bits == 8) return 4;
    const long long tiles = gemm_tiles(M, N, 8);
    const long long ktiles = (K + kGemmBK - 1) / kGemmBK;
    const long long per_cu = tiles * ktiles / num_cu;
    return tiles >= num_cu || (2 * tiles >= num_cu && per_cu >= 64) || per_cu >= 128 ? 8 : 4;
}

//  * 256-row tiles: 2 x tiles workgroups (a split tile has two or three
//    contributors), but at least one per CU: with few rows the tiles are
//    few (11008x4096 at M = 513 .. 768: 96), and too few workgroups leave
//    CUs idle (at M <= 256, before the 64-row tiles: 97 us with 64
//    workgroups against 54 us with 256).
//  * 64-row tiles (M <= 512): a CU runs about one 64-row k-tile per 0.35 us
//    whether it holds one workgroup or two, and every split tile costs a
//    32 KiB partial round trip. So one workgroup per CU when that gives each
//    at least 16 k-tiles, two per CU only from 32 k-tiles each, and with
//    fewer iterations 16 k-tiles a workgroup (at least one per tile).
//    Measured (us; 7B MLP shapes / 4096x4096; planned count first): M = 64
//    19.1 / 19.5 at 256 (128: 24.4 / 23.5), 4096x4096 14.9 at 128 (256:
//    17.8); M = 128 25.0 / 24.3 at 256 (512: 26.1 / 26.9); M = 256 36.9 /
//    34.9 at 512 (256: 40.3 / 38.4), 4096x4096 19.5 at 256 (512: 20.9); the
//    70B MLP layers at M <= 64 (28672 iterations) 58-62 us at 512 against
//    63-70 us at 256 or 1024.
//  * 256-column tiles (eight waves, one workgroup per CU): one per tile
//    when the tiles fill whole rounds of CUs, otherwise exactly one round
//    of num_cu workgroups sharing the tiles' k-steps (a second round of
//    stream-K workgroups only waits for the first: 4096x11008 at M = 2048,
//    344 tiles, 166 us with 256 workgroups, 184 us with 512, 188 us one per
//    tile).
int plan_gemm_workers(int M, int N, int K, int num_cu, int waves)
{
    if (num_cu <= 0) num_cu = 256;
    const long long tiles = gemm_tiles(M, N, waves);
    const long long ktiles = (K + kGemmBK - 1) / kGemmBK;
    if (waves == 8) {
        const long long rounds = (tiles + num_cu - 1) / num_cu;
        if (tiles * 10 >= rounds * num_cu * 9) return (int)tiles;
        return (int)std::min<long long>(std::min<long long>(num_cu, tiles * ktiles), Q4_GEMM_MAX_WORKERS);
    }
    const long long cap = 2LL * num_cu;
    const long long rounds = (tiles + cap - 1) / cap;
    if (tiles * 10 >= rounds * cap * 9 || tiles * 2 >= cap * 3) return (int)tiles;
    const long long iters = tiles * ktiles;
    long long w;
    if (gemm_bm(M) < kGemmBM)
        w = iters >= 32 * cap ? cap : iters >= 16LL * num_cu ? num_cu : std::max(tiles, iters / 16);
    else
        w = std::min(cap, std::max<long long>(2 * tiles, num_cu));
    w = std::min(w, iters);
    return (int)std::min<long long>(w, Q4_GEMM_MAX_WORKERS);
}

}  // namespace q4

extern "C" {

q4_status q4_last_status(void) { return q4::last_status(); }
const char* q4_last_error(void) { return q4::last_message(); }

q4_status q4_check_shape(int K, int N, int groupsize)
{
    int G;
    return q4::check_shape(K, N, groupsize, &G);
}

q4_status q4_check_shape_bits(int K, int N, int groupsize, int bits)
{
    int G;
    return q4::check_shape(K, N, groupsize, &G, bits);
}

q4_status q4_plan_actorder(const int32_t* g_idx_host, int K, int groupsize, int32_t* perm,
                           int* trivial)
{
    if (!g_idx_host || !perm || !trivial)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_plan_actorder: null pointer");
    if (K <= 0)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_plan_actorder: K=%d", K);
    int G = groupsize == -1 ? K : groupsize;
    if (G <= 0 || K % G)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_plan_actorder: groupsize=%d does not divide K=%d",
                        groupsize, K);
    return q4::plan_actorder(g_idx_host, K, G, perm, trivial);
}

int q4_plan_gemv_gather(int M, int K, int splits)
{
    if (M < 1 || M > Q4_GEMV_MAX_M || K < 1 || splits < 1 || splits > q4::kMaxSplits) return -1;
    return q4::gemv_gathers_x(M, K, splits) ? 1 : 0;
}

int q4_plan_gemm(int M, int N, int K, int num_cu)
{
    if (M < 1 || N < 1 || K < 1) return -1;
    return q4::plan_gemm_workers(M, N, K, num_cu, q4::gemm_waves(M, N, K, num_cu));
}

int q4_plan_gemm_waves(int M, int N, int K, int num_cu)
{
    if (M < 1 || N < 1 || K < 1) return -1;
    return q4::gemm_waves(M, N, K, num_cu);
}

q4_status q4_plan_gemv(int M, int K, int N, int groupsize, int num_cu, int* col_tiles, int* splits)
{
    if (!col_tiles || !splits) return q4::fail(Q4_ERR_INVALID_ARG, "q4_plan_gemv: null pointer");
    int G;
    q4_status st = q4::check_shape(K, N, groupsize, &G);
    if (st != Q4_OK) return st;
    if (M < 1 || M > Q4_GEMV_MAX_M)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_plan_gemv: M=%d outside [1, %d]", M, Q4_GEMV_MAX_M);
    q4::plan_gemv(M, K, N, G, num_cu, col_tiles, splits);
    return Q4_OK;
}

}  // extern "C"
