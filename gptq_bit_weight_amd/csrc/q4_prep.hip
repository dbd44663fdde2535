// Make-time repack, act-order activation permute and the debug dequant dump.
//
// Repack ("runtime initialization can ... prepack tiles, shuffle
// scales/zeros", GPTQModel wiki "Inference Backends", section "Packing,
// conversion, and runtime initialization"): qweight is rewritten once into
// the kernels' private nibble order (q4_device.h) and, for act-order, with
// its rows in the order of one stable argsort of g_idx (same page, section
// "Runtime cache lifetime"), so that every group becomes a contiguous run of
// groupsize rows. The size stays K/8 x N words.
//
// Act-order activations ("Implementation: Predibase Lorax GPTQ Exllama V1",
// Description: a scratch buffer reorders activations in the act-order case):
// x'[m, k'] = x[m, perm[k']] puts the activations in the same sorted order.
#include "q4_device.h"
#include "q4_internal.h"

namespace {

using namespace q4dev;

// One thread per output word (r', n): gather the eight codes of sorted rows
// k' = 8r' .. 8r'+7 from their original rows perm[k'] and store them in the
// private nibble slots.
__global__ __launch_bounds__(256) void q4_repack_kernel(const uint32_t* __restrict__ src,
                                                        const int32_t* __restrict__ perm,
                                                        uint32_t* __restrict__ dst, int K, int N)
{
    const size_t total = (size_t)(K / 8) * N;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int r = (int)(idx / N), n = (int)(idx % N);
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int kk = 8 * r + i;
            const int k = perm ? perm[kk] : kk;
            const uint32_t code = (src[(size_t)(k >> 3) * N + n] >> (4 * (k & 7))) & 0xFu;
            w |= code << (4 * slot_of(i));
        }
        dst[idx] = w;
    }
}

// x'[m][k'] = x[m][perm[k']]
__global__ __launch_bounds__(256) void q4_permute_x_kernel(const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ perm,
                                                           uint16_t* __restrict__ xp, int M, int K)
{
    const size_t total = (size_t)M * K;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const size_t m = idx / K;
        const int k = (int)(idx % K);
        xp[idx] = x[m * K + perm[k]];
    }
}

// Debug dump: w[k][n] (original row order) = the dequantized weight (k, n) as
// each kernel forms it, rounded to fp16. FACTORED (skinny kernel): the
// kernel's own (q - z) from sub_zero_word times the fp32 scale, which is the
// exact weight the kernel applies, then one RNE rounding. Otherwise (GEMM):
// the fp16 value dequant_word feeds to the MFMA.
template <bool FACTORED>
__global__ __launch_bounds__(256) void q4_dump_kernel(const uint32_t* __restrict__ qweight,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint32_t* __restrict__ qzeros,
                                                      const int32_t* __restrict__ inv_perm,
                                                      uint16_t* __restrict__ w, int K, int N, int G)
{
    const size_t total = (size_t)K * N;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int k = (int)(idx / N), n = (int)(idx % N);
        const int kk = inv_perm ? inv_perm[k] : k;       // sorted position of row k
        const int g = kk / G;
        const uint32_t word = qweight[(size_t)(kk >> 3) * N + n];
        const uint32_t z = (qzeros[(size_t)g * (N >> 3) + (n >> 3)] >> (4 * (n & 7))) & 0xFu;
        const uint16_t sb = scales[(size_t)g * N + n];
        if (FACTORED) {
            const h8 d = sub_zero_word(word, zero_pair(z));
            w[idx] = f32_to_f16_bits(f16_bits_to_f32(sb) * static_cast<float>(d[kk & 7]));
        } else {
            const h8 v = dequant_word(word, zero_pair(z), scale_pair(sb));
            w[idx] = bitcast<uint16_t>(v[kk & 7]);
        }
    }
}

int grid_for(size_t total)
{
    size_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

}  // namespace

namespace q4 {

hipError_t launch_repack(const uint32_t* src, const int32_t* perm, uint32_t* dst, int K, int N,
                         hipStream_t stream)
{
    hipLaunchKernelGGL(q4_repack_kernel, dim3(grid_for((size_t)(K / 8) * N)), dim3(256), 0, stream,
                       src, perm, dst, K, N);
    return hipGetLastError();
}

hipError_t launch_permute_x(const uint16_t* x, const int32_t* perm, uint16_t* xp, int M, int K,
                            hipStream_t stream)
{
    hipLaunchKernelGGL(q4_permute_x_kernel, dim3(grid_for((size_t)M * K)), dim3(256), 0, stream, x,
                       perm, xp, M, K);
    return hipGetLastError();
}

hipError_t launch_dump(const q4_matrix* h, int path, uint16_t* w, hipStream_t stream)
{
    const dim3 grid(grid_for((size_t)h->K * h->N));
    if (path == Q4_PATH_GEMV)
        hipLaunchKernelGGL(q4_dump_kernel<true>, grid, dim3(256), 0, stream, h->qweight, h->scales,
                           h->qzeros, h->inv_perm, w, h->K, h->N, h->G);
    else
        hipLaunchKernelGGL(q4_dump_kernel<false>, grid, dim3(256), 0, stream, h->qweight, h->scales,
                           h->qzeros, h->inv_perm, w, h->K, h->N, h->G);
    return hipGetLastError();
}

}  // namespace q4
