// Internal declarations shared by the host and device sources of libq4.
#pragma once

#include <cstddef>
#include <cstdint>
#include <mutex>
#include <vector>

#include "q4.h"

namespace q4 {

// ---- private weight layout -------------------------------------------------
// The packed weights are stored in k-blocks of 128 rows. Inside block b, the
// 16-byte chunk (b, kb, n) (kb = 0..3) holds four words of column n; word i of
// it packs rows 32 * (4b + i) + 8 * kb .. +7. One 16-byte load gives a lane
// the eight rows it feeds to an MFMA lane in each of four consecutive 32-row
// k-steps, and the 64 rows a prefill k-tile needs are 8 contiguous bytes of
// every chunk. Block b holds 4N chunks; inside it the columns go in tiles of
// 16, each tile's chunks ordered [kb][column] (chunk_in_block), so the 64
// lanes of a skinny-kernel wave (16 columns x 4 kb) read 1 KiB of contiguous
// memory with one instruction. (Ordering the block [kb][n] instead makes that
// read four 256-byte pieces N * 16 bytes apart; a read-only probe of the
// 7B- and 70B-shaped layers streamed 8-11% slower that way.) K is padded to a
// whole block with code 0 (the kernels give those rows zero activations).
//
// 8-bit weights use the same blocks with 32-byte chunks: word 2i + h of chunk
// (b, kb, n) holds rows 32 * (4b + i) + 8 * kb + 4h .. +3, one byte each in k
// order. A skinny-kernel lane then loads its block with two 16-byte loads,
// and a prefill k-tile (k-steps 2t, 2t + 1 of a block) is 16 contiguous bytes
// of a chunk.
constexpr int kBlockK = 128;
constexpr int num_kblocks(int K) { return (K + kBlockK - 1) / kBlockK; }
constexpr size_t packed_words(int K, int N, int bits = 4)
{
    return (size_t)num_kblocks(K) * (kBlockK * bits / 32) * (size_t)N;
}

// Chunk (b, kb, n) counted from the start of block b, for a layout of N
// columns (0 <= n < N): the tile of 16 columns holding n starts at chunk
// 4 * (n - n % 16) and is tw = min(16, N - (n - n % 16)) columns wide (the last
// tile of an N that is not a multiple of 16 is narrower).
__host__ __device__ constexpr uint32_t chunk_in_block(int kb, int n, int N)
{
    return (uint32_t)(4 * (n & ~15) + kb * ((N - (n & ~15)) < 16 ? (N - (n & ~15)) : 16) + (n & 15));
}

// ---- skinny (M <= 32) kernel geometry ------------------------------------
constexpr int kGemvMaxM = Q4_GEMV_MAX_M;   // rows the skinny kernel takes (two blocks of 16)
constexpr int kGemvWaves = 8;        // waves per workgroup (they split its K range)
constexpr int kGemvDepth = 4;        // k-blocks in flight per wave
constexpr int kMaxSplits = 16;       // K splits across workgroups (grid.y)
constexpr int kMaxColTiles = 4;      // 16-column MFMA tiles per wave
constexpr int kMaxParts = 64;        // layers one q4_make_cat handle may concatenate
// Act-order layers: when K is not split and M <= kGemvXMaxM, each workgroup
// of the skinny kernel stages all of x[:, perm] in LDS itself if K (padded to
// whole blocks) is at most kGemvXRows rows (kGemvXUnits 8-row units per
// thread) and the M rows, each padded by kGemvXPad halfs, fit in
// kGemvXLdsHalfs halfs (40 KiB); otherwise a separate kernel permutes x
// first. (Every workgroup repeats the staging, so its cost grows with M: at
// M = 4 it measured no faster than the separate permute.)
constexpr int kGemvXMaxM = 2;
constexpr int kGemvXUnits = 3;
constexpr int kGemvXRows = kGemvXUnits * 8 * 64 * kGemvWaves;
constexpr int kGemvXPad = 8;
constexpr int kGemvXLdsHalfs = 20480;

// ---- prefill (MFMA GEMM) kernel geometry ---------------------------------
constexpr int kGemmBM = 256;
constexpr int kGemmBN = 128;   // columns with four waves (256 with eight)
constexpr int kGemmBK = 64;
// The streaming GEMM takes 64-row output tiles when M <= kGemmSmallM (few
// rows: 256-row tiles leave most CUs idle and multiply padding; measured on
// the 7B MLP shapes, 64-row tiles are faster up to M = 384 (22-26% there),
// within -2 .. +7% at 512 and 5-12% slower from 768 on), else 256-row tiles.
constexpr int kGemmSmallM = 512;
inline int gemm_bm(int M) { return M <= kGemmSmallM ? 64 : kGemmBM; }
// Output tiles of an M x N product with `waves` waves (32 columns each) per
// workgroup: kGemmBN = 128 columns with four, 256 with eight.
inline int gemm_tiles(int M, int N, int waves = 4)
{
    const int bm = gemm_bm(M), bn = 32 * waves;
    return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}

// Error reporting (thread-local status + message).
q4_status fail(q4_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
q4_status last_status();
const char* last_message();

q4_status check_shape(int K, int N, int groupsize, int* G_out, int bits = 4);
q4_status plan_actorder(const int32_t* g_idx, int K, int G, int32_t* perm, int* trivial);
// Skinny-kernel launch plan: 16-column tiles per wave (1, 2 or 4) and K
// splits across workgroups (1..kMaxSplits) for a chip of num_cu CUs.
void plan_gemv(int M, int K, int N, int G, int num_cu, int* col_tiles, int* splits, int bits = 4);
// Whether the automatic dispatch runs the skinny kernel for M rows (every
// M it takes, 1 <= M <= kGemvMaxM: it measured faster than the GEMM there).
bool gemv_serves(int M, int K, int N, int G, int bits = 4);
// Whether the skinny kernel stages act-order activations itself for this
// M, K and number of K splits.
bool gemv_gathers_x(int M, int K, int splits);
// Waves per workgroup of the streaming GEMM (4: 128-column tiles, 8:
// 256-column tiles, only with 256-row tiles) for an M x N output, K rows
// and `bits`-bit weights.
int gemm_waves(int M, int N, int K, int num_cu, int bits = 4);
// Workgroups of the streaming GEMM with `waves` waves each for an M x N
// output and K rows on a chip of num_cu CUs: gemm_tiles(M, N, waves) (one
// per output tile) when the tiles fill whole rounds of the workgroups the
// CUs hold at once, otherwise a stream-K split.
int plan_gemm_workers(int M, int N, int K, int num_cu, int waves = 4);

}  // namespace q4

// The handle. Device buffers are owned; the workspace is shared by the
// handle's calls (ordered on one stream by contract).
struct q4_matrix {
    int K = 0, N = 0, G = 0, ng = 0;
    int act_order = 0;
    int bits = 4;                  // 4 or 8
    int device = -1;
    int num_cu = 256;
    uint32_t* qweight = nullptr;   // packed_words(K, N, bits): private block layout (above)
    // One device allocation holds every buffer below but the grown
    // workspaces (256-byte aligned regions, in this order).
    void* block = nullptr;
    size_t block_bytes = 0;
    // both kernels' group parameters, one word per (group, column): scale
    // bits | zero point << 16, built at make time from the checkpoint's
    // scales and packed zeros (which the handle does not keep)
    uint32_t* sz = nullptr;        // [ng][N]
    int32_t* perm = nullptr;       // [K] sorted-order -> original row, act-order only
    int32_t* inv_perm = nullptr;   // [K] original row -> sorted position, act-order only
    uint16_t* inv16 = nullptr;     // the same in 16 bits, when K <= kGemvXRows
    // skinny-kernel split-K workspace: fp32 partial sums of splits x M rows
    // (row stride M), sized at make time for the largest splits x M the plan
    // gives at any M the skinny kernel serves (none for most layers), grown
    // on demand for an explicit larger count; and arrival counters
    mutable float* partials = nullptr;     // partial_rows x N
    mutable int partial_rows = 0;
    mutable std::vector<float*> partials_grown;   // allocated on demand, freed with the handle
    uint32_t* counters = nullptr;  // [ceil(N / 16)]: one per column tile at the narrowest tiling
    // act-order activation workspace, grown on demand: x[:, perm] as fp16 [M][K]
    mutable std::mutex ws_mutex;
    mutable uint16_t* xperm = nullptr;
    mutable size_t xperm_elems = 0;
    mutable std::vector<uint16_t*> xperm_retired;   // outgrown buffers, freed with the handle
};
