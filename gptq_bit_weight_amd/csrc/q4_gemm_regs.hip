// Prefill fused W4A16 GEMM (M > 16), register-staged variant.
//
// This variant suits grids with at least two output tiles per CU: its 80 KiB
// of LDS lets two workgroups share a CU, whose waves hide each other's
// latencies. (The direct-to-LDS pipelined variant in q4_gemm.hip uses nearly
// all of the LDS for one workgroup and wins when tiles are scarce.)
//
// The multiply itself is a dense contraction, so it runs on
// v_mfma_f32_32x32x16_f16 with fp32 accumulation (GPTQModel wiki "Inference
// Backends", hardware table, ExLlama v2 row: FP32 accumulation, FP16 scales).
// The weight tile is staged in LDS still packed (4 bits per weight) and each
// wave dequantizes the words it feeds to the MFMA in registers, so no fp16
// weight tile is ever written to device memory ("GPTQ's 'Exllama Kernel Not
// Installed' Warning", section "What the fallback actually does").
//
// Tiling: a workgroup of 4 waves (2 x 2) computes a BM x BN = 256 x 128
// output tile; each wave owns 128 x 64 (4 x 2 MFMA tiles of 32 x 32), so every
// dequantized word feeds 4 MFMAs and the vector ALU stays well under the
// matrix pipe. K advances in BK = 64 rows: the activation tile (256 x 64 fp16,
// row stride padded to 72 halfs so 16-byte LDS reads of 8 consecutive rows
// hit distinct banks) and the packed weight tile (8 x 128 words) are
// double-buffered in LDS; the next tile's global loads are in flight while
// the current one is multiplied. A k-tile's packed words are 8 contiguous
// bytes of each 16-byte chunk (kb, n) of the private layout (words 2h, 2h + 1
// of k-block b for k-tile 2b + h); in LDS they are stored as [kb][h'][n], so
// tile row r (rows 8r .. 8r+7 of the tile) is row (r & 3) * 2 + (r >> 2).
//
// Global loads are bounds-checked raw buffer loads (out-of-range offsets
// read zeros), so ragged M, N and K need no branches.
//
// Workgroup order: when the row tiles divide evenly over the 8 XCDs (the
// round-robin dispatch puts workgroup i on XCD i % 8), every XCD works on its
// own row tiles, so each XCD's L2 keeps its activation rows resident while
// the packed weights stream through; otherwise row-major order.
#include "q4_device.h"
#include "q4_internal.h"

namespace {

using namespace q4dev;

constexpr int BM = q4::kGemmBM;
constexpr int BN = q4::kGemmBN;
constexpr int BK = q4::kGemmBK;
constexpr int AST = BK + 8;          // LDS row stride of the activation tile (halfs)
constexpr int NT = q4::kGemmThreads;
constexpr int WTM = BM / 2;          // wave tile rows
constexpr int WTN = BN / 2;          // wave tile columns
constexpr int MI = WTM / 32;         // 32x32 MFMA tiles per wave along M
constexpr int NJ = WTN / 32;         // ... along N
constexpr int A_LOADS = BM * BK / 8 / NT;    // 16-byte activation loads per thread per tile
static_assert(BN * BK / 8 / 4 == NT, "two 8-byte (two-word) weight loads per thread per tile");

struct GemmArgs {
    const uint32_t* qweight;
    const uint16_t* scales;
    const uint32_t* qzeros;
    const uint16_t* x;
    const uint16_t* bias;
    uint16_t* out;
    int M, K, N, G;
};

struct TileRegs {
    u4 a[A_LOADS];
    u2 b[2];       // words (2h, 2h + 1) of chunk (kb, n), n = two adjacent columns
};

// Scales/zeros of the NJ columns a lane multiplies, for up to two groups of a
// k-tile (groups of 32 rows).
struct GroupRegs {
    uint32_t s[2][NJ];
    uint32_t z[2][NJ];
};

struct Lane {
    uint32_t a_off[A_LOADS];   // activation byte offsets (k0 = 0)
    uint32_t a_kc;             // k offset (rows) of this thread's activation chunks
    uint32_t b_off[2];         // weight byte offsets of the two chunks (k-tile 0)
    uint32_t b_kill[2];        // kOOB for a column past N
    uint32_t s_off[NJ];        // scale byte offsets (group 0)
    uint32_t z_off[NJ];        // zero-word byte offsets (group 0)
    uint32_t z_shift[NJ];
};

template <int NG>
__device__ __forceinline__ void load_tile(TileRegs& t, GroupRegs& gr, const GemmArgs& p,
                                          const Lane& ln, rsrc_t rx, rsrc_t rw, rsrc_t rs,
                                          rsrc_t rz, int k0)
{
    const uint32_t a_kill = (ln.a_kc + (uint32_t)k0 < (uint32_t)p.K) ? 0u : kOOB;
#pragma unroll
    for (int e = 0; e < A_LOADS; ++e) t.a[e] = buf_load16(rx, ln.a_off[e] + (uint32_t)k0 * 2u + a_kill);
    const uint32_t tile_off = (uint32_t)(k0 >> 7) * (uint32_t)p.N * 64u + 8u * (uint32_t)((k0 >> 6) & 1);
#pragma unroll
    for (int v = 0; v < 2; ++v) t.b[v] = buf_load8(rw, (ln.b_off[v] + tile_off) | ln.b_kill[v]);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const int k = k0 + 32 * gi;
        const uint32_t g = (uint32_t)(min(k, p.K - 1) / p.G);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            gr.s[gi][j] = buf_load2(rs, ln.s_off[j] + g * (uint32_t)p.N * 2u);
            gr.z[gi][j] = buf_load4(rz, ln.z_off[j] + g * (uint32_t)(p.N >> 3) * 4u);
        }
    }
}

__device__ __forceinline__ void store_tile(const TileRegs& t, uint16_t* As, uint32_t* Bs, int tid)
{
#pragma unroll
    for (int e = 0; e < A_LOADS; ++e) {
        const int c = tid + NT * e;
        const int row = c >> 3, kc = c & 7;
        *reinterpret_cast<u4*>(As + row * AST + 8 * kc) = t.a[e];
    }
    const int kb = tid >> 6, n = 2 * (tid & 63);
    *reinterpret_cast<u2*>(Bs + (2 * kb) * BN + n) = u2{t.b[0][0], t.b[1][0]};
    *reinterpret_cast<u2*>(Bs + (2 * kb + 1) * BN + n) = u2{t.b[0][1], t.b[1][1]};
}

template <int NG>
__global__ __launch_bounds__(NT) void q4_gemm_regs_kernel(GemmArgs p)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * AST];
    __shared__ __attribute__((aligned(16))) uint32_t Bs[2][(BK / 8) * BN];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, lhi = lane >> 5;

    // Tile order (see the header).
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

    const rsrc_t rx = make_rsrc(p.x, (uint32_t)p.M * (uint32_t)p.K * 2u);
    const rsrc_t rw = make_rsrc(p.qweight, (uint32_t)q4::num_kblocks(p.K) * (uint32_t)p.N * 64u);
    const int ng = p.K / p.G;
    const rsrc_t rs = make_rsrc(p.scales, (uint32_t)ng * (uint32_t)p.N * 2u);
    const rsrc_t rz = make_rsrc(p.qzeros, (uint32_t)ng * (uint32_t)(p.N >> 3) * 4u);

    Lane ln;
    ln.a_kc = 8u * (uint32_t)(tid & 7);
#pragma unroll
    for (int e = 0; e < A_LOADS; ++e) {
        const int row = (tid + NT * e) >> 3;
        ln.a_off[e] = ((uint32_t)(m0 + row) * (uint32_t)p.K + ln.a_kc) * 2u;   // rows >= M fall outside x
    }
#pragma unroll
    for (int v = 0; v < 2; ++v) {
        const int kb = tid >> 6, n = n0 + 2 * (tid & 63) + v;
        ln.b_off[v] = q4::chunk_in_block(kb, min(n, p.N - 1), p.N) * 16u;
        ln.b_kill[v] = n < p.N ? 0u : kOOB;
    }
    int lane_cols[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int n = n0 + wn * WTN + 32 * j + l32;
        lane_cols[j] = n;
        const uint32_t kill = n < p.N ? 0u : kOOB;
        ln.s_off[j] = (uint32_t)n * 2u + kill;
        ln.z_off[j] = (uint32_t)(n >> 3) * 4u + kill;
        ln.z_shift[j] = 4u * (uint32_t)(n & 7);
    }

    f16x acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int ktiles = (p.K + BK - 1) / BK;
    TileRegs tr;
    GroupRegs gcur, gnext;
    load_tile<NG>(tr, gcur, p, ln, rx, rw, rs, rz, 0);
    store_tile(tr, As[0], Bs[0], tid);
    __syncthreads();

    for (int kt = 0; kt < ktiles; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < ktiles;
        if (more) load_tile<NG>(tr, gnext, p, ln, rx, rw, rs, rz, (kt + 1) * BK);
        __builtin_amdgcn_sched_barrier(0);

        zero_t hz[NG][NJ];
        h2 s2[NG][NJ];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                hz[gi][j] = zero_pair((gcur.z[gi][j] >> ln.z_shift[j]) & 0xFu);
                s2[gi][j] = scale_pair(gcur.s[gi][j]);
            }

        const uint16_t* A = As[buf];
        const uint32_t* B = Bs[buf];
        const int k0 = kt * BK;
#pragma unroll
        for (int sub = 0; sub < BK / 16; ++sub) {
            if (k0 + 16 * sub < p.K) {
                const int gi = NG == 2 ? (sub >> 1) : 0;
                h8 b[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                {
                    const int r = 2 * sub + lhi;   // tile row
                    b[j] = dequant_word(B[((r & 3) * 2 + (r >> 2)) * BN + wn * WTN + 32 * j + l32],
                                        hz[gi][j], s2[gi][j]);
                }
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    const h8 a = *reinterpret_cast<const h8*>(A + (wm * WTM + 32 * i + l32) * AST +
                                                              16 * sub + 8 * lhi);
#pragma unroll
                    for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32(a, b[j], acc[i][j]);
                }
            }
        }
        if (more) {
            store_tile(tr, As[buf ^ 1], Bs[buf ^ 1], tid);
            gcur = gnext;
        }
        __syncthreads();
    }

    // Epilogue: fp32 bias, one round-to-nearest-even cast, store. Lane l holds
    // rows 8*(r/4) + 4*(l/32) + r%4 of column l%32 of each 32 x 32 tile.
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int n = lane_cols[j];
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

hipError_t launch_gemm_regs(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
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
    // Groups of 64 rows or more never straddle a 64-row k-tile; groups of 32
    // change once inside it.
    if (h->G % BK != 0 && h->G != h->K)
        hipLaunchKernelGGL(q4_gemm_regs_kernel<2>, dim3(tiles), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL(q4_gemm_regs_kernel<1>, dim3(tiles), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace q4
