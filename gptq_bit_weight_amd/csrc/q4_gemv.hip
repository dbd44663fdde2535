// Skinny fused W4A16 kernel for 1 <= M <= 16 (decode).
//
// Weight-bound decoding is limited by memory bandwidth ("GPTQ's 'Exllama
// Kernel Not Installed' Warning", section "What the fallback actually
// does"), so the kernel streams the packed words once with 16-byte loads,
// dequantizes them in registers and never writes a dequantized weight.
//
// Mapping (one workgroup = 4 waves = 64 output columns x a K range):
//  * lane l owns columns c = tile*64 + 4*(l % 16) .. +3 (one 16-byte load of
//    four consecutive words of a qweight row) and k-block kb = l / 16 of
//    every 32-row k-step: rows 32t + 8kb .. +7, i.e. word row 4t + kb;
//  * per k-step each lane feeds four v_mfma_f32_16x16x32_f16, one per owned
//    column: A = activations (row m = l % 16, zero for m >= M), B = the eight
//    values q - z of one word, exact small integers in fp16. M is padded to
//    16 on the matrix pipe, which has the capacity to spare; the vector ALU
//    is the scarce unit here, so the per-group scale is applied once per
//    group to the fp32 group sum: sum_k x*s*(q - z) = s * sum_k x*(q - z)
//    (the weight s*(q - z) is exact in fp32, so this is the product with the
//    exact dequantized weight, accumulated in fp32);
//  * the four waves split the workgroup's K range; their fp32 results are
//    summed in LDS in wave order;
//  * grid.y splits K across workgroups when there are few column tiles. Each
//    split writes fp32 partials; the last workgroup of a column tile to
//    arrive (counted with an agent-scope atomic) sums them in split order, so
//    the result does not depend on timing. Reductions stay in fp32 (GPTQModel
//    wiki "Inference Backends", section "Numeric epilogues": FP32 split/tile
//    reductions, bias added before the single cast).
#include "q4_device.h"
#include "q4_internal.h"

namespace {

using namespace q4dev;

struct GemvArgs {
    const uint32_t* qweight;
    const uint16_t* scales;
    const uint32_t* qzeros;
    const uint16_t* x;
    const uint16_t* bias;
    uint16_t* out;
    float* partials;
    uint32_t* counters;
    int M, K, N, G;
    int gshift;          // group of k-step t = t >> gshift (31 for a single group)
    int splits;
    int batches_per_split;
    int batches_per_wave;
};

constexpr int kSteps = q4::kBatchSteps;    // k-steps per batch

// Per-lane constants of the load addressing (byte offsets inside each tensor;
// an invalid column carries kOOB so every load of it returns zeros).
struct LaneAddr {
    uint32_t w;     // qweight: kb-th word row of a k-step, the lane's 4 columns
    uint32_t x;     // x: row m, k-block kb
    uint32_t s;     // scales: the lane's 4 columns
    uint32_t z;     // qzeros: the word holding the lane's columns
    uint32_t zshift;
};

struct Rsrc {
    rsrc_t w, x, s, z;
};

// One batch of loads for one lane: kSteps k-steps of weights and activations
// plus the scales/zeros they need. Every load is unconditional; k-steps past
// the end of K read zeros (weights and activations alike).
//
// GS = k-steps per group: 1, 2 (groups of 32, 64 rows), 4, 8 (128, 256) or 0
// (one group over K). Batches start at multiples of 4 k-steps, so with GS >= 4
// (or 0) a batch lies in one group.
template <int GS>
struct Batch {
    static constexpr int NG = GS == 1 ? 4 : GS == 2 ? 2 : 1;
    u4 w[kSteps];
    u4 a[kSteps];
    u2 s[NG];
    uint32_t z[NG];
};

template <int GS>
__device__ __forceinline__ void load_batch(Batch<GS>& b, const GemvArgs& p, const Rsrc& r,
                                           const LaneAddr& la, int batch)
{
    const int ksteps = p.K >> 5;
    const int t0 = batch * kSteps;
    const uint32_t row_bytes = (uint32_t)p.N * 4u;
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const int t = t0 + i;
        const uint32_t kill = t < ksteps ? 0u : kOOB;
        b.w[i] = buf_load16(r.w, la.w + (uint32_t)(4 * t) * row_bytes + kill);
        b.a[i] = buf_load16(r.x, la.x + (uint32_t)t * 64u + kill);
    }
#pragma unroll
    for (int gi = 0; gi < Batch<GS>::NG; ++gi) {
        const int t = t0 + gi * (kSteps / Batch<GS>::NG);
        const uint32_t g = GS == 0 ? 0u : (uint32_t)(t >> p.gshift);
        const uint32_t kill = t < ksteps ? 0u : kOOB;
        b.s[gi] = buf_load8(r.s, la.s + g * (uint32_t)p.N * 2u + kill);
        b.z[gi] = buf_load4(r.z, la.z + g * (uint32_t)(p.N >> 3) * 4u + kill);
    }
}

// Multiply one batch into the group sums `acc` and fold finished groups into
// `tot`: tot += s * acc (fp32). FRESH: the batch starts a group (acc restarts
// from zero); FOLD: the batch ends a group. Only GS = 8 and GS = 0 decide
// these per batch; smaller groups start and end inside every batch.
template <int GS, bool FRESH, bool FOLD>
__device__ __forceinline__ void compute_batch(const Batch<GS>& b, f4 acc[4], f4 tot[4],
                                              uint32_t zshift)
{
    h2 hz[4];
    float sf[4];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        constexpr int per = GS == 1 ? 1 : GS == 2 ? 2 : kSteps;   // k-steps per group in a batch
        const bool starts = (i % per) == 0;
        const bool fresh = starts && (GS == 1 || GS == 2 || GS == 4 || FRESH);
        const bool ends = (i % per) == per - 1;
        const bool fold = ends && (GS == 1 || GS == 2 || GS == 4 || FOLD);
        if (starts) {
            const int gi = i / per;
            const uint32_t z4 = b.z[gi] >> zshift;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hz[j] = zero_pair((z4 >> (4 * j)) & 0xFu);
                sf[j] = f16_bits_to_f32((uint16_t)(b.s[gi][j >> 1] >> (16 * (j & 1))));
            }
        }
        const h8 a = bitcast<h8>(b.a[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[j] = mfma16(a, sub_zero_word(b.w[i][j], hz[j]), fresh ? f4{0.f, 0.f, 0.f, 0.f} : acc[j]);
        if (fold) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) tot[j][e] = __builtin_fmaf(sf[j], acc[j][e], tot[j][e]);
        }
    }
}

template <int GS>
__device__ __forceinline__ void compute_any(const Batch<GS>& b, f4 acc[4], f4 tot[4], uint32_t zshift,
                                            bool fresh, bool fold)
{
    if (GS == 8 || GS == 0) {
        if (fresh && fold) compute_batch<GS, true, true>(b, acc, tot, zshift);
        else if (fresh) compute_batch<GS, true, false>(b, acc, tot, zshift);
        else if (fold) compute_batch<GS, false, true>(b, acc, tot, zshift);
        else compute_batch<GS, false, false>(b, acc, tot, zshift);
    } else {
        compute_batch<GS, true, true>(b, acc, tot, zshift);
    }
}

template <int GS>
__global__ __launch_bounds__(256) void q4_gemv_kernel(GemvArgs p)
{
    __shared__ float red[q4::kWaves][16][q4::kColTile];
    __shared__ int last_flag;

    const int tid = threadIdx.x;
    // The wave index is uniform across the wave; saying so keeps the batch
    // bookkeeping in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int kb = lane >> 4;
    const int m = lane & 15;
    const int col = blockIdx.x * q4::kColTile + 4 * (lane & 15);
    const bool col_ok = col < p.N;
    const int ksteps = p.K >> 5;
    const int total_batches = (ksteps + kSteps - 1) / kSteps;
    const int ng = p.K / p.G;

    Rsrc r;
    r.w = make_rsrc(p.qweight, (uint32_t)(p.K >> 3) * (uint32_t)p.N * 4u);
    r.x = make_rsrc(p.x, (uint32_t)p.M * (uint32_t)p.K * 2u);
    r.s = make_rsrc(p.scales, (uint32_t)ng * (uint32_t)p.N * 2u);
    r.z = make_rsrc(p.qzeros, (uint32_t)ng * (uint32_t)(p.N >> 3) * 4u);
    LaneAddr la;
    const uint32_t col_kill = col_ok ? 0u : kOOB;
    la.w = ((uint32_t)kb * (uint32_t)p.N + (uint32_t)col) * 4u + col_kill;
    la.x = ((uint32_t)m * (uint32_t)p.K + 8u * kb) * 2u;     // rows m >= M fall outside x
    la.s = (uint32_t)col * 2u + col_kill;
    la.z = (uint32_t)(col >> 3) * 4u + col_kill;
    la.zshift = 4u * (col & 7);

    const int split = blockIdx.y;
    const int b_split0 = split * p.batches_per_split;
    const int b_split1 = min(b_split0 + p.batches_per_split, total_batches);
    const int b0 = b_split0 + wave * p.batches_per_wave;
    const int b1 = min(b0 + p.batches_per_wave, b_split1);

    f4 acc[4], tot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc[j] = f4{0.f, 0.f, 0.f, 0.f};
        tot[j] = f4{0.f, 0.f, 0.f, 0.f};
    }

    if (b0 < b1) {
        // Two register buffers: the loads of batch b+1 are in flight while
        // batch b is unpacked and multiplied. The prefetch index is clamped
        // to the wave's last batch (a repeated load, never out of range).
        // sched_barrier keeps the compiler from sinking the prefetch below
        // the arithmetic it is meant to overlap.
        Batch<GS> A, B;
        load_batch(A, p, r, la, b0);
        for (int b = b0; b < b1; b += 2) {
            load_batch(B, p, r, la, min(b + 1, b1 - 1));
            __builtin_amdgcn_sched_barrier(0);
            compute_any(A, acc, tot, la.zshift, b == b0 || (GS == 8 && (b & 1) == 0),
                        b + 1 == b1 || (GS == 8 && (b & 1) == 1));
            if (b + 1 >= b1) break;
            load_batch(A, p, r, la, min(b + 2, b1 - 1));
            __builtin_amdgcn_sched_barrier(0);
            compute_any(B, acc, tot, la.zshift, GS == 8 && ((b + 1) & 1) == 0,
                        b + 2 == b1 || (GS == 8 && ((b + 1) & 1) == 1));
        }
    }

    // Cross-wave reduction. Lane l holds rows 4*(l/16) + i of the columns
    // 4*(l%16) + j (16x16 MFMA output layout).
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            red[wave][4 * kb + i][4 * (lane & 15) + j] = tot[j][i];
    __syncthreads();

    const int n_elems = p.M * q4::kColTile;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int idx = tid + 256 * e;
        v[e] = 0.f;
        if (idx < n_elems) {
            const int r = idx / q4::kColTile, c = idx % q4::kColTile;
            v[e] = ((red[0][r][c] + red[1][r][c]) + red[2][r][c]) + red[3][r][c];
        }
    }

    const int tile_col0 = blockIdx.x * q4::kColTile;
    if (p.splits == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = tid + 256 * e;
            const int r = idx / q4::kColTile, c = tile_col0 + idx % q4::kColTile;
            if (idx < n_elems && c < p.N) {
                float y = v[e];
                if (p.bias) y += f16_bits_to_f32(p.bias[c]);
                p.out[(size_t)r * p.N + c] = f32_to_f16_bits(y);
            }
        }
        return;
    }

    // Split-K: publish this split's partial sums, then let the last arriver
    // of the column tile reduce all splits in split order. The partials are
    // written and read with agent-scope atomic accesses, which go to the
    // device-coherent level directly; the only ordering needed is that every
    // wave's stores are complete before the arrival count is bumped. (A full
    // __threadfence() would write back and invalidate the whole L2 of the
    // XCD, once per workgroup, which serializes across the chip.)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int idx = tid + 256 * e;
        const int r = idx / q4::kColTile, c = tile_col0 + idx % q4::kColTile;
        if (idx < n_elems && c < p.N)
            __hip_atomic_store(&p.partials[((size_t)split * 16 + r) * p.N + c], v[e], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&p.counters[blockIdx.x], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        last_flag = (prev == (uint32_t)(p.splits - 1));
    }
    __syncthreads();
    if (!last_flag) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int idx = tid + 256 * e;
        const int r = idx / q4::kColTile, c = tile_col0 + idx % q4::kColTile;
        if (idx < n_elems && c < p.N) {
            float y = 0.f;
            for (int s = 0; s < p.splits; ++s)
                y += __hip_atomic_load(&p.partials[((size_t)s * 16 + r) * p.N + c], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            if (p.bias) y += f16_bits_to_f32(p.bias[c]);
            p.out[(size_t)r * p.N + c] = f32_to_f16_bits(y);
        }
    }
    if (tid == 0)
        __hip_atomic_store(&p.counters[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

namespace q4 {

hipError_t launch_gemv(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
                       int M, int splits, hipStream_t stream)
{
    GemvArgs p;
    p.qweight = h->qweight;
    p.scales = h->scales;
    p.qzeros = h->qzeros;
    p.x = x;
    p.bias = bias;
    p.out = out;
    p.partials = h->partials;
    p.counters = h->counters;
    p.M = M;
    p.K = h->K;
    p.N = h->N;
    p.G = h->G;
    p.gshift = 31;
    for (int sh = 0; sh < 30; ++sh)
        if ((32 << sh) == h->G && h->G != h->K) p.gshift = sh;
    const int ksteps = h->K / 32;
    const int total_batches = (ksteps + kBatchSteps - 1) / kBatchSteps;
    p.splits = splits;
    p.batches_per_split = (total_batches + splits - 1) / splits;
    p.batches_per_wave = (p.batches_per_split + kWaves - 1) / kWaves;
    dim3 grid((h->N + kColTile - 1) / kColTile, splits);
    // k-steps per group: a batch spans 4 k-steps starting at a multiple of 4,
    // so groups of 128 or 256 rows never straddle a batch; one group over K
    // (per-channel) never changes at all.
    const int gs = h->G == h->K ? 0 : h->G / 32;
    switch (gs) {
    case 1: hipLaunchKernelGGL(q4_gemv_kernel<1>, grid, dim3(256), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(q4_gemv_kernel<2>, grid, dim3(256), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(q4_gemv_kernel<4>, grid, dim3(256), 0, stream, p); break;
    case 8: hipLaunchKernelGGL(q4_gemv_kernel<8>, grid, dim3(256), 0, stream, p); break;
    case 0: hipLaunchKernelGGL(q4_gemv_kernel<0>, grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace q4
