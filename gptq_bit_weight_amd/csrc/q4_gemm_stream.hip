// Prefill fused GPTQ GEMM (M > 16) on the matrix cores: activations staged
// in LDS, weights streamed into registers.
//
// q4_gemm_stream_kernel<NG, KT, BF, W8>: NG groups per 64-row k-tile (2 for
// groups of 32), KT (K not a multiple of 64), BF (bfloat16 activations and
// output), W8 (8-bit codes).
//
// The multiply runs on v_mfma_f32_32x32x16_f16 with fp32 accumulation
// (GPTQModel wiki "Inference Backends", hardware table, ExLlama v2 row: FP32
// accumulation, FP16 scales). The packed weights never touch LDS: every wave
// loads the words of its own columns straight into registers, one k-tile
// ahead, and dequantizes them there for the MFMA, so no dequantized weight
// exists anywhere but in registers ("GPTQ's 'Exllama Kernel Not Installed'
// Warning", section "What the fallback actually does").
//
// Tiling: a workgroup of 4 waves (2 x 2) computes a 256 x 128 output tile;
// each wave owns 128 x 64 (4 x 2 MFMA tiles of 32 x 32). K advances in
// 64-row tiles.
//  * Activations: a 2-stage LDS ring (32 KiB a stage, 16-byte chunks of the
//    128-byte rows XOR-swizzled by (row / 2) % 8) filled by direct-to-LDS
//    buffer loads. 64 KiB of LDS lets two workgroups share a CU.
//  * Weights: for its two columns a lane needs, per k-tile, words 2h and
//    2h + 1 of chunks (b, kb) and (b, kb + 2) of the private block layout
//    (k-tile 2b + h, kb = lane / 32): two 8-byte loads per column. With the
//    scale and zero words of the tile's group(s), these go to one of two
//    register sets; the k-loop is unrolled by two so that the set a step
//    multiplies is never a set a load is filling.
//  * One barrier per k-tile: after it, every wave has finished the previous
//    tile, so the stage that tile used is refilled (tile kt + 1) while tile
//    kt is multiplied.
//  * W8: 8-bit codes. A chunk is 32 bytes (two words per k-step), so a
//    column's k-tile is 16 contiguous bytes of chunks (b, kb) and (b, kb + 2):
//    two 16-byte loads instead of two 8-byte ones.
//  * BF: bfloat16 activations, bias and output (the activation dtype is kept;
//    GPTQModel wiki "Inference Backends", hardware table, ExLlama v2 row). The
//    matrix pipe then takes bfloat16 operands: each weight s * (q - z) is
//    formed exactly in fp32 and rounded once to bfloat16.
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
constexpr int A_TILE_BYTES = BM * BK * 2;          // 32 KiB
constexpr int A_LOADS = A_TILE_BYTES / (NT * 16);  // 8 direct loads per thread
static_assert(BK == 64 && BN == 128 && NT == 256 && NJ == 2, "index arithmetic below assumes these");

typedef __attribute__((address_space(3))) void lds_void;

struct GemmArgs {
    const uint32_t* qweight;
    const uint16_t* scales;
    const uint32_t* qzeros;
    const uint16_t* x;
    const uint16_t* bias;
    uint16_t* out;
    int M, K, N, G;
    int zrow;               // bytes per row of packed zeros (N * bits / 8)
};

__device__ __forceinline__ uint32_t swz(int r, int c) { return (uint32_t)(r * 128 + ((c ^ ((r >> 1) & 7)) << 4)); }

#define Q4S_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One k-tile of a lane's weights: w[j][0] = words (2h, 2h+1) of chunk
// (b, kb, n_j) -- sub-steps 0 and 2 -- and w[j][1] those of chunk
// (b, kb + 2, n_j) -- sub-steps 1 and 3; scale and zero words of the tile's
// NG groups (two for groups of 32 rows).
template <int NG, bool W8>
struct BRegs {
    std::conditional_t<W8, u4, u2> w[NJ][2];
    uint32_t s[NG][NJ];
    uint32_t z[NG][NJ];
};

struct Ctx {
    rsrc_t rx, rw, rs, rz;
    uint32_t a_off[A_LOADS];   // activation byte offsets for k0 = 0 (rows >= M fall outside x)
    uint32_t a_k[A_LOADS];     // k of each chunk for k0 = 0
    uint32_t w_off[NJ][2];     // weight byte offsets of the two chunks per column (k-tile 0)
    uint32_t s_off[NJ];        // scale byte offsets (group 0)
    uint32_t z_off[NJ];        // zero-word byte offsets (group 0)
    uint32_t z_shift[NJ];
};

// The k offset of the tile is wave-uniform (a scalar register); rows past M
// lie past the end of x through the per-lane offset alone. Only with KT can a
// chunk lie past K (in the last tile); its lanes are pushed out of range.
template <bool KT>
__device__ __forceinline__ void load_a(const Ctx& c, const GemmArgs& p, char* stage, int wave, int kt)
{
    const uint32_t k0 = (uint32_t)kt * BK;
#pragma unroll
    for (int e = 0; e < A_LOADS; ++e) {
        const uint32_t kill = (!KT || c.a_k[e] + k0 < (uint32_t)p.K) ? 0u : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rx, (lds_void*)(stage + (e * 4 + wave) * 1024), 16,
                                                 (int)(c.a_off[e] + kill), (int)(k0 * 2u), 0, 0);
    }
}

template <int NG, bool W8>
__device__ __forceinline__ void load_b(BRegs<NG, W8>& R, const Ctx& c, const GemmArgs& p, int kt)
{
    constexpr uint32_t CB = W8 ? 32 : 16;   // chunk bytes
    const uint32_t tile = (uint32_t)(kt >> 1) * (uint32_t)p.N * 4u * CB + (CB / 2) * (uint32_t)(kt & 1);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            if constexpr (W8) R.w[j][v] = buf_load16(c.rw, c.w_off[j][v], tile);
            else R.w[j][v] = buf_load8(c.rw, c.w_off[j][v], tile);
        }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const int k = min(kt * BK + 32 * gi, p.K - 1);
        const uint32_t g = (uint32_t)(k / p.G);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            R.s[gi][j] = buf_load2(c.rs, c.s_off[j], g * (uint32_t)p.N * 2u);
            R.z[gi][j] = buf_load4(c.rz, c.z_off[j], g * (uint32_t)p.zrow);
        }
    }
}

// KT: K is not a multiple of 64, so the last k-tile skips its sub-steps past
// K (a separate instantiation, so that the common kernel has no branch
// around the multiply: the accumulators stay in the same registers).
// (Two workgroups per CU: the register budget is 256 per lane.)
template <int NG, bool KT, bool BF, bool W8>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2))) void q4_gemm_stream_kernel(GemmArgs p)
{
    __shared__ __attribute__((aligned(1024))) char lds_a0[A_TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_a1[A_TILE_BYTES];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, lhi = lane >> 5;

    // Workgroup order: when the row tiles divide evenly over the 8 XCDs
    // (workgroup i runs on XCD i % 8), every XCD works on its own row tiles
    // and keeps their activations in its L2; otherwise row-major order.
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
    c.rw = make_rsrc(p.qweight, (uint32_t)q4::num_kblocks(p.K) * (uint32_t)p.N * (W8 ? 128u : 64u));
    c.rs = make_rsrc(p.scales, (uint32_t)ng * (uint32_t)p.N * 2u);
    c.rz = make_rsrc(p.qzeros, (uint32_t)ng * (uint32_t)p.zrow);
#pragma unroll
    for (int e = 0; e < A_LOADS; ++e) {
        // instruction e of wave w fills rows 8 * (4e + w) .. +7 of the stage;
        // lane i lands in slot i % 8 of row i / 8, which holds chunk
        // slot ^ ((row >> 1) & 7)
        const int row = 8 * (4 * e + wave) + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        c.a_k[e] = 8u * (uint32_t)chunk;
        c.a_off[e] = ((uint32_t)(m0 + row) * (uint32_t)p.K + c.a_k[e]) * 2u;
    }
    int lane_cols[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        lane_cols[j] = n0 + wn * WTN + 32 * j + l32;
        const uint32_t n = (uint32_t)min(lane_cols[j], p.N - 1);   // columns past N are never stored
#pragma unroll
        for (int v = 0; v < 2; ++v) c.w_off[j][v] = ((uint32_t)(lhi + 2 * v) * (uint32_t)p.N + n) * (W8 ? 32u : 16u);
        c.s_off[j] = n * 2u;
        c.z_off[j] = (n >> (W8 ? 2 : 3)) * 4u;
        c.z_shift[j] = W8 ? 8u * (n & 3u) : 4u * (n & 7u);
    }

    f16x acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int ktiles = (p.K + BK - 1) / BK;
    BRegs<NG, W8> R0, R1;

    // Multiply k-tile kt: activations from `A`, weights from register set R.
    // With KT, sub-steps past K (zero activations) are skipped so that their
    // weights (code 0, any scale) add nothing.
    auto mma = [&](const char* A, const BRegs<NG, W8>& R, int kt) {
        zero_t hz[NG][NJ];
        h2 s2[NG][NJ];
        mix_t mz[NJ];   // BF: the constants of the current group only (registers)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if constexpr (!BF) {
                    hz[gi][j] = zero_pair((R.z[gi][j] >> c.z_shift[j]) & (W8 ? 0xFFu : 0xFu));
                    s2[gi][j] = scale_pair(R.s[gi][j]);
                }
            }
        const int k0 = kt * BK;
#pragma unroll
        for (int sub = 0; sub < BK / 16; ++sub) {
            const int gi = NG == 2 ? (sub >> 1) : 0;
            if constexpr (BF) {
                if (sub % (4 / NG) == 0)
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        mz[j] = mix_consts((R.z[gi][j] >> c.z_shift[j]) & (W8 ? 0xFFu : 0xFu),
                                           f16_bits_to_f32((uint16_t)R.s[gi][j]));
            }
            if (!KT || k0 + 16 * sub < p.K) {
                u4 b[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if constexpr (W8) {
                        // sub-step s: words 2 (s / 2), 2 (s / 2) + 1 of the 16 bytes from chunk s % 2
                        const uint32_t w0 = R.w[j][sub & 1][2 * (sub >> 1)], w1 = R.w[j][sub & 1][2 * (sub >> 1) + 1];
                        if constexpr (BF) b[j] = bitcast<u4>(mix_word8(w0, w1, mz[j]));
                        else b[j] = bitcast<u4>(dequant_word8(w0, w1, hz[gi][j], s2[gi][j]));
                    } else {
                        const uint32_t w = R.w[j][sub & 1][sub >> 1];
                        if constexpr (BF) b[j] = bitcast<u4>(mix_word(w, mz[j]));
                        else b[j] = bitcast<u4>(dequant_word(w, hz[gi][j], s2[gi][j]));
                    }
                }
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    const u4 a = *reinterpret_cast<const u4*>(A + swz(wm * WTM + 32 * i + l32, 2 * sub + lhi));
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        if constexpr (BF) acc[i][j] = mfma32(bitcast<b8>(a), bitcast<b8>(b[j]), acc[i][j]);
                        else acc[i][j] = mfma32(bitcast<h8>(a), bitcast<h8>(b[j]), acc[i][j]);
                    }
                }
            }
        }
    };

    // One k-tile on stage S with register set Rc, prefetching tile kt + 1
    // (clamped: past the end it reloads the last tile, into buffers nobody
    // reads again) into the other stage and set Rn.
    auto step = [&](auto S_tag, int kt, BRegs<NG, W8>& Rc, BRegs<NG, W8>& Rn) {
        constexpr int S = decltype(S_tag)::value;
        char* cur = S == 0 ? lds_a0 : lds_a1;
        char* nxt = S == 0 ? lds_a1 : lds_a0;
        // Tile kt's activations and weight registers, the only loads in
        // flight, must have landed (the activations in every thread's part of
        // the stage). The wait names no count, so it holds whatever order the
        // compiler issued the two kinds of loads in.
        Q4S_VMCNT(0);
        lds_barrier();
        const int kn = min(kt + 1, ktiles - 1);
        load_a<KT>(c, p, nxt, wave, kn);
        load_b(Rn, c, p, kn);
        mma(cur, Rc, kt);
    };

    load_a<KT>(c, p, lds_a0, wave, 0);
    load_b(R0, c, p, 0);
    int kt = 0;
    for (; kt + 1 < ktiles; kt += 2) {
        step(std::integral_constant<int, 0>{}, kt, R0, R1);
        step(std::integral_constant<int, 1>{}, kt + 1, R1, R0);
    }
    if (kt < ktiles) step(std::integral_constant<int, 0>{}, kt, R0, R1);
    // Drain the last (unused) prefetch before the workgroup's LDS is reused.
    Q4S_VMCNT(0);

    // Epilogue: fp32 bias, one round-to-nearest-even cast, store. Lane l holds
    // rows 8*(r/4) + 4*(l/32) + r%4 of column l%32 of each 32 x 32 tile.
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int n = lane_cols[j];
        if (n >= p.N) continue;
        const float bv = p.bias ? act_to_f32<BF>(p.bias[n]) : 0.f;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * WTM + 32 * i + 8 * (r >> 2) + 4 * lhi + (r & 3);
                if (m < p.M) p.out[(size_t)m * p.N + n] = f32_to_act<BF>(acc[i][j][r] + bv);
            }
    }
}

template <bool BF, bool W8>
hipError_t launch_stream(const GemmArgs& p, int tiles, bool g32, bool kt, hipStream_t stream)
{
    if (g32 && kt)
        hipLaunchKernelGGL((q4_gemm_stream_kernel<2, true, BF, W8>), dim3(tiles), dim3(NT), 0, stream, p);
    else if (g32)
        hipLaunchKernelGGL((q4_gemm_stream_kernel<2, false, BF, W8>), dim3(tiles), dim3(NT), 0, stream, p);
    else if (kt)
        hipLaunchKernelGGL((q4_gemm_stream_kernel<1, true, BF, W8>), dim3(tiles), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((q4_gemm_stream_kernel<1, false, BF, W8>), dim3(tiles), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

namespace q4 {

hipError_t launch_gemm_stream(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
                              int M, bool bf16, hipStream_t stream)
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
    const bool g32 = h->G % BK != 0 && h->G != h->K, kt = h->K % BK != 0;
    p.zrow = h->N * h->bits / 8;
    if (h->bits == 8)
        return bf16 ? launch_stream<true, true>(p, tiles, g32, kt, stream)
                    : launch_stream<false, true>(p, tiles, g32, kt, stream);
    return bf16 ? launch_stream<true, false>(p, tiles, g32, kt, stream)
                : launch_stream<false, false>(p, tiles, g32, kt, stream);
}

}  // namespace q4
