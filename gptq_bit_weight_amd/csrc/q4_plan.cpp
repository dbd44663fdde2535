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
q4_status check_shape(int K, int N, int groupsize, int* G_out)
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
    // Byte offsets inside the packed weights stay below 2^31 (the kernels mark
    // out-of-range lanes by adding 2^31).
    if ((long long)K * (long long)N / 2 > (1LL << 31) - 1)
        return fail(Q4_ERR_UNSUPPORTED, "K*N/2 = %lld bytes of packed weights exceeds 2^31 - 1",
                    (long long)K * (long long)N / 2);
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

// Split-K plan of the skinny kernel. One workgroup covers kColTile columns and
// a contiguous K range that its four waves divide; splits add workgroups
// along K when the column tiles alone cannot fill the chip. Each split costs
// a round of fp32 partial sums (8 * splits * M * N bytes) and puts the
// last-arriver reduction on the critical path, so splits only grow while the
// grid stays within kTargetWorkgroups and every wave keeps at least
// kMinBatchesPerWave batches. (Measured on MI355X at M = 1..16 over the
// Llama-7B and Llama-70B layer shapes.)
int plan_splits(int M, int K, int N, int G)
{
    if (M <= 0 || K <= 0 || N <= 0 || K % 32) return 0;
    (void)G;
    const int col_tiles = (N + kColTile - 1) / kColTile;
    const int batches = (K / 32 + kBatchSteps - 1) / kBatchSteps;
    int s = 1;
    while (2 * s <= kMaxSplits && col_tiles * 2 * s <= kTargetWorkgroups &&
           batches >= 2 * s * kWaves * kMinBatchesPerWave)
        s *= 2;
    return s;
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

int q4_plan_splits(int M, int K, int N, int groupsize)
{
    int G;
    if (M <= 0 || q4::check_shape(K, N, groupsize, &G) != Q4_OK) return 0;
    return q4::plan_splits(M, K, N, G);
}

}  // extern "C"
