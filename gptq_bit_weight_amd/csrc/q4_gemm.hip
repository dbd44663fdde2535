// Prefill fused W4A16 GEMM (M > 16) on the matrix cores: direct-to-LDS
// pipelined variant.
//
// The multiply itself is a dense contraction, so it runs on
// v_mfma_f32_32x32x16_f16 with fp32 accumulation (GPTQModel wiki "Inference
// Backends", hardware table, ExLlama v2 row: FP32 accumulation, FP16 scales).
// The weights travel from memory to LDS still packed (4 bits per weight);
// each workgroup dequantizes its packed tile once into an fp16 tile in LDS,
// which the matrix cores read. No fp16 weight tile is ever written to device
// memory ("GPTQ's 'Exllama Kernel Not Installed' Warning", section "What the
// fallback actually does").
//
// Tiling: a workgroup of 4 waves (2 x 2) computes a BM x BN = 256 x 128
// output tile; each wave owns 128 x 64 (4 x 2 MFMA tiles of 32 x 32). K
// advances in BK = 64 rows per tile.
//
// Data movement per k-tile (all global reads are bounds-checked raw buffer
// loads that write straight into LDS, so ragged M, N and K need no branches
// and no registers carry the tiles):
//  * activations (256 x 64 fp16) and packed weights (8 x 128 words plus the
//    tile's scale and zero rows) each use a ring of 3 LDS stages and are
//    loaded 2 tiles ahead. A k-tile's packed words are 8 contiguous bytes of
//    each 16-byte chunk (kb, n) of the private layout (words i = 2h, 2h + 1
//    of k-block b for k-tile 2b + h); they land in LDS as [kb][n][2], and
//    tile row r (rows 8r .. 8r+7 of the tile) is word r >> 2 of chunk r & 3. Each stage is its own __shared__ array and the
//    k-loop is unrolled by 3, so the compiler can see that the LDS reads of
//    one stage never alias the loads landing in another and does not wait
//    for them;
//  * while the waves multiply tile t, every thread dequantizes 4 packed words
//    of tile t+1 (one column, 32 rows of one group) into the next fp16 weight
//    tile (a third ring of 3), so each weight is unpacked once per workgroup.
// LDS rows of 64 fp16 (128 bytes) are stored with the 16-byte chunk c of row
// r at slot c ^ ((r >> 1) & 7): a 16-byte read is served 16 lanes at a time,
// and 16 consecutive rows at one chunk then cover all 64 banks exactly once.
//
// Workgroup order: when the row tiles divide evenly over the 8 XCDs (the
// round-robin dispatch puts workgroup i on XCD i % 8), every XCD works on its
// own row tiles, so each XCD's L2 keeps its activation rows resident while
// the packed weights stream through; otherwise row-major order.
#include <type_traits>

#include "q4_device.h"
#include "q4_internal.h"

namespace {

using namespace q4dev;

constexpr int BM = q4::kGemmBM;      // 256
constexpr int BN = q4::kGemmBN;      // 128
constexpr int BK = q4::kGemmBK;      // 64
constexpr int NT = q4::kGemmThreads; // 256
constexpr int WTM = BM / 2;          // wave tile rows
constexpr int WTN = BN / 2;          // wave tile columns
constexpr int MI = WTM / 32;
constexpr int NJ = WTN / 32;
constexpr int STAGES = 3;
constexpr int A_TILE_BYTES = BM * BK * 2;          // 32 KiB
constexpr int BP_WORD_BYTES = (BK / 8) * BN * 4;   // 4 KiB of packed words
constexpr int BP_SZ_BYTES = 256;                    // one row of scales or zero words
constexpr int BP_TILE_BYTES = BP_WORD_BYTES + 4 * BP_SZ_BYTES;   // + scales/zeros of 2 groups
constexpr int B16_TILE_BYTES = BN * BK * 2;        // 16 KiB
constexpr int A_LOADS = A_TILE_BYTES / (NT * 16);  // 8 direct loads per thread
constexpr int BP_LOADS = BP_WORD_BYTES / (NT * 4);  // 4-byte packed-word loads per thread
constexpr int B_LOADS = BP_LOADS + 1;               // + one scale or zero-word load
static_assert(BP_LOADS == 4, "one packed-word load per chunk row kb");
static_assert(BK == 64 && BN == 128 && NT == 256, "index arithmetic below assumes these");

typedef __attribute__((address_space(3))) void lds_void;

struct GemmArgs {
    const uint32_t* qweight;
    const uint16_t* scales;
    const uint32_t* qzeros;
    const uint16_t* x;
    const uint16_t* bias;
    uint16_t* out;
    int M, K, N, G;
};

// Byte offset of 16-byte chunk c of row r in a swizzled 64-fp16-per-row tile.
__device__ __forceinline__ uint32_t swz(int r, int c) { return (uint32_t)(r * 128 + ((c ^ ((r >> 1) & 7)) << 4)); }

// Wait until at most n vector-memory loads of this wave are outstanding
// (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at
// their maxima, i.e. not waited for).
#define Q4_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

__device__ __forceinline__ void wait_vm(int n)
{
    switch (n) {
    case A_LOADS: Q4_VMCNT(A_LOADS); break;
    case A_LOADS + B_LOADS: Q4_VMCNT(A_LOADS + B_LOADS); break;
    case 2 * A_LOADS + B_LOADS: Q4_VMCNT(2 * A_LOADS + B_LOADS); break;
    default: Q4_VMCNT(0); break;
    }
}

// Workgroup barrier for the LDS pipeline. __syncthreads() also waits for
// every outstanding vector-memory load (its release fence covers the
// direct-to-LDS loads still in flight), which would drain the pipeline; the
// waits this pipeline needs are issued explicitly before the barrier (vmcnt
// for the stages about to be read, lgkmcnt for this thread's LDS writes).
// The "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct Ctx {
    rsrc_t rx, rw, rs, rz;
    uint32_t a_off[A_LOADS];   // activation byte offsets for k0 = 0 (rows >= M fall outside x)
    uint32_t a_k[A_LOADS];     // k of each chunk for k0 = 0
    uint32_t bp_off;           // packed-weight byte offset of this lane's word in k-tile 0, kb = 0
    uint32_t bp_kbs;           // bytes from chunk (kb, n) to chunk (kb + 1, n): 16 * tile width
    uint32_t bp_kill;          // kOOB for a column past N
    uint32_t sz_off;           // scale or zero-word byte offset of this lane (row 0, kill folded in)
    bool sz_is_zero;           // this wave loads zero words (else scales)
    int sz_group;              // 0: first group of the tile, 1: second (groups of 32 rows)
};

// Direct-to-LDS loads of activation tile kt into the stage `dst_stage`
// (A_LOADS per thread).
__device__ __forceinline__ void load_a(const Ctx& c, const GemmArgs& p, char* dst_stage, int wave, int kt)
{
    const uint32_t k0 = (uint32_t)kt * BK;
#pragma unroll
    for (int e = 0; e < A_LOADS; ++e) {
        const uint32_t kill = (c.a_k[e] + k0 < (uint32_t)p.K) ? 0u : kOOB;
        char* dst = dst_stage + (e * 4 + wave) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rx, (lds_void*)dst, 16, (int)(c.a_off[e] + k0 * 2u + kill), 0, 0, 0);
    }
}

// Direct-to-LDS loads of packed tile kt into stage st: the packed words (one
// 4-byte load per chunk row kb per thread; instruction kb of wave w fills
// 256 bytes of the [kb][n][2] layout) and one row of scales or zero words
// per wave (B_LOADS loads per thread).
__device__ __forceinline__ void load_b(const Ctx& c, const GemmArgs& p, char* base, int wave, int kt)
{
    const uint32_t tile_off = (uint32_t)(kt >> 1) * (uint32_t)p.N * 64u + 8u * (uint32_t)(kt & 1);
#pragma unroll
    for (int kb = 0; kb < BP_LOADS; ++kb)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            c.rw, (lds_void*)(base + (kb * 4 + wave) * 256), 4,
            (int)((c.bp_off + (uint32_t)kb * c.bp_kbs + tile_off) | c.bp_kill), 0, 0, 0);
    const int k = kt * BK + 32 * c.sz_group;
    const uint32_t kill = k < p.K ? 0u : kOOB;
    const uint32_t g = (uint32_t)(min(k, p.K - 1) / p.G);
    char* dst = base + BP_WORD_BYTES + (2 * c.sz_group + (c.sz_is_zero ? 1 : 0)) * BP_SZ_BYTES;
    if (c.sz_is_zero)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rz, (lds_void*)dst, 4,
                                                 (int)(c.sz_off + g * (uint32_t)(p.N >> 3) * 4u + kill), 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rs, (lds_void*)dst, 4,
                                                 (int)(c.sz_off + g * (uint32_t)p.N * 2u + kill), 0, 0, 0);
}

// Dequantize this thread's 4 packed words of a tile (column n, word rows
// r0..r0+3, all in one group) into the fp16 tile.
__device__ __forceinline__ void dequant_tile(const char* bp, char* b16, int n, int r0, int k0, int K)
{
    const int gi = r0 >> 2;   // which of the tile's two group rows (equal unless groups of 32)
    const uint16_t sb = reinterpret_cast<const uint16_t*>(bp + BP_WORD_BYTES + (2 * gi) * BP_SZ_BYTES)[n];
    const uint32_t zw = reinterpret_cast<const uint32_t*>(bp + BP_WORD_BYTES + (2 * gi + 1) * BP_SZ_BYTES)[n >> 3];
    const zero_t hz = zero_pair((zw >> (4 * (n & 7))) & 0xFu);
    const h2 s2 = scale_pair(sb);
    const uint32_t* words = reinterpret_cast<const uint32_t*>(bp);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = r0 + i;
        h8 v = dequant_word(words[((r & 3) * BN + n) * 2 + (r >> 2)], hz, s2);
        if (k0 + 8 * r >= K) v = h8{0, 0, 0, 0, 0, 0, 0, 0};     // rows past K (tail tile)
        // The fp16 weight tiles are never targets of the direct-to-LDS loads,
        // but the compiler cannot prove that for a computed address and would
        // wait for every load in flight before this store; it is issued as
        // inline asm instead. (LDS operations complete in order, so the
        // compiler's own lgkmcnt waits stay correct with one more in flight.)
        const uint32_t addr = (uint32_t)(uintptr_t)(b16 + swz(n, r));
        asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v));
    }
}

__global__ __launch_bounds__(NT) void q4_gemm_dma_kernel(GemmArgs p)
{
    __shared__ __attribute__((aligned(1024))) char lds_a0[A_TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_a1[A_TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_a2[A_TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_bp0[BP_TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_bp1[BP_TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_bp2[BP_TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_w0[B16_TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_w1[B16_TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_w2[B16_TILE_BYTES];
    // Stage I of each ring, chosen at compile time so that every LDS access
    // names its __shared__ array directly.
    auto stage_a = [&](auto I) -> char* {
        if constexpr (decltype(I)::value == 0) return lds_a0;
        else if constexpr (decltype(I)::value == 1) return lds_a1;
        else return lds_a2;
    };
    auto stage_b = [&](auto I) -> char* {
        if constexpr (decltype(I)::value == 0) return lds_bp0;
        else if constexpr (decltype(I)::value == 1) return lds_bp1;
        else return lds_bp2;
    };
    auto stage_w = [&](auto I) -> char* {
        if constexpr (decltype(I)::value == 0) return lds_w0;
        else if constexpr (decltype(I)::value == 1) return lds_w1;
        else return lds_w2;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, lhi = lane >> 5;

    const int nt = (p.N + BN - 1) / BN, mt = (p.M + BM - 1) / BM;
    const int id = blockIdx.x;
    int mtile, ntile;
    if (mt % 8 == 0) {
        const int xcd = id & 7, r = id >> 3;
        mtile = (r / nt) * 8 + xcd;
        ntile = r % nt;
    } else {
        mtile = id / nt;
        ntile = id % nt;
    }
    const int m0 = mtile * BM, n0 = ntile * BN;

    Ctx c;
    const int ng = p.K / p.G;
    c.rx = make_rsrc(p.x, (uint32_t)p.M * (uint32_t)p.K * 2u);
    c.rw = make_rsrc(p.qweight, (uint32_t)q4::num_kblocks(p.K) * (uint32_t)p.N * 64u);
    c.rs = make_rsrc(p.scales, (uint32_t)ng * (uint32_t)p.N * 2u);
    c.rz = make_rsrc(p.qzeros, (uint32_t)ng * (uint32_t)(p.N >> 3) * 4u);
#pragma unroll
    for (int e = 0; e < A_LOADS; ++e) {
        // instruction e of wave w fills rows 8*(4e + w) .. +7 of the stage;
        // lane i lands in slot i % 8 of row i / 8, which holds chunk
        // slot ^ ((row >> 1) & 7) (see swz)
        const int row = 8 * (4 * e + wave) + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        c.a_k[e] = 8u * (uint32_t)chunk;
        c.a_off[e] = ((uint32_t)(m0 + row) * (uint32_t)p.K + c.a_k[e]) * 2u;
    }
    {
        // packed tile: lane pair (2i, 2i + 1) of wave w takes the two words of
        // column n0 + 32w + i
        const int col = n0 + 32 * wave + (lane >> 1);
        const int cn = min(col, p.N - 1);
        c.bp_off = q4::chunk_in_block(0, cn, p.N) * 16u + 4u * (uint32_t)(lane & 1);
        c.bp_kbs = (q4::chunk_in_block(1, cn, p.N) - q4::chunk_in_block(0, cn, p.N)) * 16u;
        c.bp_kill = col < p.N ? 0u : kOOB;
    }
    {
        // scales/zeros: waves 0/1 load the scale / zero row of the tile's first
        // group, waves 2/3 those of its second group (groups of 32 rows)
        c.sz_is_zero = (wave & 1) != 0;
        c.sz_group = wave >> 1;
        if (c.sz_is_zero) {
            const int col = n0 + 8 * lane;          // zero word lane -> columns col .. col+7
            c.sz_off = (uint32_t)(col >> 3) * 4u + (lane < 16 && col < p.N ? 0u : kOOB);
        } else {
            const int col = n0 + 2 * lane;          // scale pair lane -> columns col, col+1
            c.sz_off = (uint32_t)col * 2u + (col < p.N ? 0u : kOOB);
        }
    }
    // dequant assignment: column dq_n of the tile, word rows dq_r0 .. dq_r0+3
    const int dq_n = tid & (BN - 1);
    const int dq_r0 = 4 * (tid >> 7);

    f16x acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int ktiles = (p.K + BK - 1) / BK;

    // Prologue: tiles 0 and 1 in flight (packed first, then activations);
    // packed tile 0 dequantized.
    load_b(c, p, stage_b(I0{}), wave, 0);
    load_a(c, p, stage_a(I0{}), wave, 0);
    if (ktiles > 1) {
        load_b(c, p, stage_b(I1{}), wave, 1);
        load_a(c, p, stage_a(I1{}), wave, 1);
    }
    Q4_VMCNT(0);
    lds_barrier();
    dequant_tile(stage_b(I0{}), stage_w(I0{}), dq_n, dq_r0, 0, p.K);

    // One k-tile: S = kt % 3 is a compile-time stage index.
    auto step = [&](auto S_tag, int kt) {
        constexpr int S = decltype(S_tag)::value;
        using IS = std::integral_constant<int, S>;
        using IS1 = std::integral_constant<int, (S + 1) % STAGES>;
        using IS2 = std::integral_constant<int, (S + 2) % STAGES>;
        // Issue tile kt+2: packed first, then activations.
        int n_cur = 0;
        if (kt + 2 < ktiles) {
            // the waits below count loads in this order: keep it
            __builtin_amdgcn_sched_barrier(0);
            load_b(c, p, stage_b(IS2{}), wave, kt + 2);
            __builtin_amdgcn_sched_barrier(0);
            load_a(c, p, stage_a(IS2{}), wave, kt + 2);
            __builtin_amdgcn_sched_barrier(0);
            n_cur = A_LOADS + B_LOADS;
        }
        // This step reads activation tile kt (issued two steps ago) and packed
        // tile kt+1 (issued one step ago, before that step's activations):
        // the activation loads of tile kt+1 and this step's loads may remain.
        wait_vm((kt + 1 < ktiles ? A_LOADS : 0) + n_cur);
        lds_barrier();

        const char* A = stage_a(IS{});
        const char* B = stage_w(IS{});
        const int k0 = kt * BK;
        // Rows past K hold zeros in both tiles (activation loads past K are
        // out of range; the dequant writes zeros there), so the last tile
        // needs no special case. The dequant of tile kt+1 runs unconditionally
        // (past the last tile it fills a buffer nobody reads).
        // The operands of 16-row sub-step s + 1 are read from LDS while the
        // matrix cores work on sub-step s (two register sets), so the LDS
        // latency hides behind the MFMAs of the one wave per SIMD.
        h8 fa[2][MI], fb[2][NJ];
        auto read_frag = [&](int f, int sub) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                fb[f][j] = *reinterpret_cast<const h8*>(B + swz(wn * WTN + 32 * j + l32, 2 * sub + lhi));
#pragma unroll
            for (int i = 0; i < MI; ++i)
                fa[f][i] = *reinterpret_cast<const h8*>(A + swz(wm * WTM + 32 * i + l32, 2 * sub + lhi));
        };
        read_frag(0, 0);
#pragma unroll
        for (int sub = 0; sub < BK / 16; ++sub) {
            if (sub + 1 < BK / 16) read_frag((sub + 1) & 1, sub + 1);
            if (sub == 1) {
                // dequantize packed tile kt+1 while the matrix cores run
                dequant_tile(stage_b(IS1{}), stage_w(IS1{}), dq_n, dq_r0, k0 + BK, p.K);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32(fa[sub & 1][i], fb[sub & 1][j], acc[i][j]);
        }
        lds_barrier();
    };
    for (int kt = 0; kt < ktiles; kt += STAGES) {
        step(std::integral_constant<int, 0>{}, kt);
        if (kt + 1 < ktiles) step(std::integral_constant<int, 1>{}, kt + 1);
        if (kt + 2 < ktiles) step(std::integral_constant<int, 2>{}, kt + 2);
    }

    // Epilogue: fp32 bias, one round-to-nearest-even cast, store. Lane l holds
    // rows 8*(r/4) + 4*(l/32) + r%4 of column l%32 of each 32 x 32 tile.
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int n = n0 + wn * WTN + 32 * j + l32;
        if (n >= p.N) continue;
        const float bv = p.bias ? f16_bits_to_f32(p.bias[n]) : 0.f;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * WTM + 32 * i + 8 * (r >> 2) + 4 * lhi + (r & 3);
                if (m < p.M) p.out[(size_t)m * p.N + n] = f32_to_f16_bits(acc[i][j][r] + bv);
            }
    }
}

}  // namespace

namespace q4 {

hipError_t launch_gemm_dma(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
                       int M, hipStream_t stream)
{
    GemmArgs p;
    p.qweight = h->qweight;
    p.scales = h->scales;
    p.qzeros = h->qzeros;
    p.x = x;
    p.bias = bias;
    p.out = out;
    p.M = M;
    p.K = h->K;
    p.N = h->N;
    p.G = h->G;
    const int tiles = ((h->N + BN - 1) / BN) * ((M + BM - 1) / BM);
    hipLaunchKernelGGL(q4_gemm_dma_kernel, dim3(tiles), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace q4
