// Prefill fused W4A16 GEMM (M > 16) on the matrix cores.
//
// The multiply itself is a dense contraction, so it runs on
// v_mfma_f32_32x32x16_f16 with fp32 accumulation (GPTQModel wiki "Inference
// Backends", hardware table, ExLlama v2 row: FP32 accumulation, FP16 scales).
// The weight tile is staged in LDS still packed (4 bits per weight) and each
// wave dequantizes the words it feeds to the MFMA in registers, so no fp16
// weight tile is ever written to device memory ("GPTQ's 'Exllama Kernel Not
// Installed' Warning", section "What the fallback actually does").
//
// Tiling: a workgroup of 4 waves computes a BM x BN = 128 x 128 output tile,
// each wave a 64 x 64 quarter (2 x 2 MFMA tiles of 32 x 32). K advances in
// BK = 64 rows: the activation tile (128 x 64 fp16) and the packed weight
// tile (8 x 128 words) are double-buffered in LDS; the next tile's global
// loads are in flight while the current one is multiplied.
#include "q4_device.h"
#include "q4_internal.h"

namespace {

using namespace q4dev;

constexpr int BM = q4::kGemmBM;
constexpr int BN = q4::kGemmBN;
constexpr int BK = q4::kGemmBK;
constexpr int AST = BK + 8;          // LDS row stride of the activation tile (halfs)
constexpr int NT = q4::kGemmThreads;

struct GemmArgs {
    const uint32_t* qweight;
    const uint16_t* scales;
    const uint32_t* qzeros;
    const uint16_t* x;
    const uint16_t* bias;
    uint16_t* out;
    int M, K, N, G;
};

// Per-thread registers holding one k-tile on its way from memory to LDS.
struct TileRegs {
    u4 a[4];     // 4 x 16 bytes of the activation tile
    u4 b;        // 16 bytes (4 words) of the packed weight tile
};

// Scales/zeros of the two columns a lane multiplies, for up to two groups.
struct GroupRegs {
    uint32_t s[2][2];
    uint32_t z[2][2];
};

template <bool STEP_GROUPS>
__device__ __forceinline__ void load_tile(TileRegs& t, GroupRegs& gr, const GemmArgs& p, int m0,
                                          int n0, int k0, int tid, int lane_cols[2])
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int c = tid + NT * e;
        const int row = c >> 3, kc = c & 7;
        const int m = m0 + row, k = k0 + 8 * kc;
        if (m < p.M && k < p.K)
            t.a[e] = *reinterpret_cast<const u4*>(p.x + (size_t)m * p.K + k);
        else
            t.a[e] = u4{0, 0, 0, 0};
    }
    {
        const int brow = tid >> 5, bcol = tid & 31;
        const int r = (k0 >> 3) + brow, n = n0 + 4 * bcol;
        if (8 * r < p.K && n < p.N)
            t.b = *reinterpret_cast<const u4*>(p.qweight + (size_t)r * p.N + n);
        else
            t.b = u4{0, 0, 0, 0};
    }
    constexpr int NG = STEP_GROUPS ? 2 : 1;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const int k = min(k0 + 32 * gi, p.K - 1);
        const int g = k / p.G;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = lane_cols[j];
            if (n < p.N) {
                gr.s[gi][j] = p.scales[(size_t)g * p.N + n];
                gr.z[gi][j] = (p.qzeros[(size_t)g * (p.N >> 3) + (n >> 3)] >> (4 * (n & 7))) & 0xFu;
            } else {
                gr.s[gi][j] = 0;
                gr.z[gi][j] = 0;
            }
        }
    }
}

__device__ __forceinline__ void store_tile(const TileRegs& t, uint16_t* As, uint32_t* Bs, int tid)
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int c = tid + NT * e;
        const int row = c >> 3, kc = c & 7;
        *reinterpret_cast<u4*>(As + row * AST + 8 * kc) = t.a[e];
    }
    const int brow = tid >> 5, bcol = tid & 31;
    *reinterpret_cast<u4*>(Bs + brow * BN + 4 * bcol) = t.b;
}

template <bool STEP_GROUPS>
__global__ __launch_bounds__(NT) void q4_gemm_kernel(GemmArgs p)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * AST];
    __shared__ __attribute__((aligned(16))) uint32_t Bs[2][(BK / 8) * BN];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int l32 = lane & 31, lhi = lane >> 5;

    int lane_cols[2] = {n0 + wn * 64 + l32, n0 + wn * 64 + 32 + l32};

    f16x acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int ktiles = (p.K + BK - 1) / BK;
    TileRegs tr;
    GroupRegs gcur, gnext;
    load_tile<STEP_GROUPS>(tr, gcur, p, m0, n0, 0, tid, lane_cols);
    store_tile(tr, As[0], Bs[0], tid);
    __syncthreads();

    for (int kt = 0; kt < ktiles; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < ktiles;
        if (more) load_tile<STEP_GROUPS>(tr, gnext, p, m0, n0, (kt + 1) * BK, tid, lane_cols);

        constexpr int NG = STEP_GROUPS ? 2 : 1;
        h2 hz[NG][2], s2[NG][2];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                hz[gi][j] = zero_pair(gcur.z[gi][j]);
                s2[gi][j] = scale_pair(gcur.s[gi][j]);
            }

        const uint16_t* A = As[buf];
        const uint32_t* B = Bs[buf];
        const int k0 = kt * BK;
#pragma unroll
        for (int sub = 0; sub < BK / 16; ++sub) {
            if (k0 + 16 * sub < p.K) {
                const int gi = STEP_GROUPS ? (sub >> 1) : 0;
                h8 a[2], b[2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    a[i] = *reinterpret_cast<const h8*>(A + (wm * 64 + 32 * i + l32) * AST + 16 * sub + 8 * lhi);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    b[j] = dequant_word(B[(2 * sub + lhi) * BN + wn * 64 + 32 * j + l32], hz[gi][j], s2[gi][j]);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
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
    for (int j = 0; j < 2; ++j) {
        const int n = lane_cols[j];
        if (n >= p.N) continue;
        const float bv = p.bias ? f16_bits_to_f32(p.bias[n]) : 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * lhi + (r & 3);
                if (m < p.M) p.out[(size_t)m * p.N + n] = f32_to_f16_bits(acc[i][j][r] + bv);
            }
    }
}

}  // namespace

namespace q4 {

hipError_t launch_gemm(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
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
    dim3 grid((h->N + BN - 1) / BN, (M + BM - 1) / BM);
    // Groups of 64 rows or more never straddle a 64-row k-tile.
    const bool step_groups = (h->G % BK) != 0 && h->G != h->K;
    if (step_groups)
        hipLaunchKernelGGL(q4_gemm_kernel<true>, grid, dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL(q4_gemm_kernel<false>, grid, dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace q4
