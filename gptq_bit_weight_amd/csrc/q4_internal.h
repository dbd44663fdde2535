// Internal declarations shared by the host and device sources of libq4.
#pragma once

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "q4.h"

namespace q4 {

// ---- skinny (M <= 16) kernel geometry ------------------------------------
constexpr int kWaves = 4;            // waves per workgroup
constexpr int kColTile = 64;         // columns per workgroup (16 lanes x 4 words)
constexpr int kBatchSteps = 4;       // k-steps (32 rows each) per unrolled batch
constexpr int kMaxSplits = 16;       // K splits (grid.y)
constexpr int kTargetWorkgroups = 256;
constexpr int kMinBatchesPerWave = 2;

// ---- prefill (MFMA GEMM) kernel geometry ---------------------------------
constexpr int kGemmBM = 256;
constexpr int kGemmBN = 128;
constexpr int kGemmBK = 64;
constexpr int kGemmThreads = 256;

// Error reporting (thread-local status + message).
q4_status fail(q4_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
q4_status last_status();
const char* last_message();

q4_status check_shape(int K, int N, int groupsize, int* G_out);
q4_status plan_actorder(const int32_t* g_idx, int K, int G, int32_t* perm, int* trivial);
int plan_splits(int M, int K, int N, int G);

}  // namespace q4

// The handle. Device buffers are owned; the workspace is shared by the
// handle's calls (ordered on one stream by contract).
struct q4_matrix {
    int K = 0, N = 0, G = 0, ng = 0;
    int act_order = 0;
    int device = -1;
    int num_cu = 256;
    uint32_t* qweight = nullptr;   // [K/8][N], nibble slots interleaved (see q4_device.h)
    uint16_t* scales = nullptr;    // [ng][N] fp16
    uint32_t* qzeros = nullptr;    // [ng][N/8]
    int32_t* perm = nullptr;       // [K] sorted-order -> original row, act-order only
    int32_t* inv_perm = nullptr;   // [K] original row -> sorted position, act-order only
    // skinny-kernel split-K workspace: partial sums and arrival counters
    float* partials = nullptr;     // [kMaxSplits][16][N]
    uint32_t* counters = nullptr;  // [ceil(N / kColTile)]
    // act-order activation workspace, grown on demand: x[:, perm] as fp16 [M][K]
    mutable std::mutex ws_mutex;
    mutable uint16_t* xperm = nullptr;
    mutable size_t xperm_elems = 0;
};
