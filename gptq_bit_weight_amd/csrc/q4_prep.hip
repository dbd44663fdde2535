// Make-time repack, act-order activation permute and the debug dequant dump.
//
// Repack (GPTQModel wiki "Inference Backends", section "Packing, conversion,
// and runtime initialization": a backend may rearrange the checkpoint's
// tiles, scales and zeros into its own layout when it initializes): qweight
// is rewritten once into
// the kernels' private layout -- 128-row k-blocks of 16-byte chunks, word i
// of chunk (b, kb, n) packing rows 32 * (4b + i) + 8 * kb .. +7 of column n,
// chunks in 16-column tiles (q4_internal.h), each word in the nibble slot order of q4_device.h -- and,
// for act-order, with its rows in the order of one stable argsort of g_idx
// (same page, section "Runtime cache lifetime"), so that every group becomes
// a contiguous run of groupsize rows. Rows past K (up to the next multiple of
// 128) hold code 0.
//
// Act-order activations ("Implementation: Predibase Lorax GPTQ Exllama V1",
// Description: a scratch buffer reorders activations in the act-order case):
// x'[m, k'] = x[m, perm[k']] puts the activations in the same sorted order.
#include "q4_device.h"
#include "q4_internal.h"

namespace {

using namespace q4dev;

// Row k' of the private layout: its chunk (b, kb), the word inside the chunk
// and the element e inside the k-step's eight rows (4-bit: word i; 8-bit:
// word 2i + e / 4).
__device__ __forceinline__ size_t private_word(int kk, int n, int N, int* e, int bits)
{
    const int b = kk >> 7, i = (kk >> 5) & 3, kb = (kk >> 3) & 3;
    *e = kk & 7;
    const size_t chunk = (size_t)b * 4 * N + q4::chunk_in_block(kb, n, N);
    if (bits == 8) return chunk * 8 + 2 * i + (*e >> 2);
    return chunk * 4 + i;
}

// One thread per output word of one part (N columns of a handle with n_total,
// placed at column col_off): gather the eight codes of (sorted) rows
// k' = 32 * (4b + i) + 8 * kb + e from their original rows perm[k'] and store
// them in the private nibble slots.
__global__ __launch_bounds__(256) void q4_repack_kernel(const uint32_t* __restrict__ src,
                                                        const int32_t* __restrict__ perm,
                                                        uint32_t* __restrict__ dst, int K, int N,
                                                        int n_total, int col_off)
{
    const size_t total = q4::packed_words(K, N, 4);
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int i = (int)(idx & 3);
        const size_t chunk = idx >> 2;
        const int n = (int)(chunk % N);
        const int q = (int)(chunk / N);                  // 4 * b + kb
        const int k0 = 32 * (4 * (q >> 2) + i) + 8 * (q & 3);
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int kk = k0 + e;
            if (kk >= K) break;
            const int k = perm ? perm[kk] : kk;
            const uint32_t code = (src[(size_t)(k >> 3) * N + n] >> (4 * (k & 7))) & 0xFu;
            w |= code << (4 * slot_of(e));
        }
        dst[((size_t)(q >> 2) * 4 * n_total + q4::chunk_in_block(q & 3, col_off + n, n_total)) * 4 + i] = w;
    }
}

// 8-bit codes: one thread per output word, word 2i + h of chunk (b, kb) =
// the four codes of (sorted) rows 32 * (4b + i) + 8 * kb + 4h + e, e = 0..3,
// in k order, gathered from original rows perm[k'] (code of row k in byte
// k % 4 of source word k / 4). Rows past K get code 0.
__global__ __launch_bounds__(256) void q4_repack8_kernel(const uint32_t* __restrict__ src,
                                                         const int32_t* __restrict__ perm,
                                                         uint32_t* __restrict__ dst, int K, int N,
                                                         int n_total, int col_off)
{
    const size_t total = q4::packed_words(K, N, 8);
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int wi = (int)(idx & 7);
        const size_t chunk = idx >> 3;
        const int n = (int)(chunk % N);
        const int q = (int)(chunk / N);                  // 4 * b + kb
        const int k0 = 32 * (4 * (q >> 2) + (wi >> 1)) + 8 * (q & 3) + 4 * (wi & 1);
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int kk = k0 + e;
            if (kk >= K) break;
            const int k = perm ? perm[kk] : kk;
            const uint32_t code = (src[(size_t)(k >> 2) * N + n] >> (8 * (k & 3))) & 0xFFu;
            w |= code << (8 * e);
        }
        dst[((size_t)(q >> 2) * 4 * n_total + q4::chunk_in_block(q & 3, col_off + n, n_total)) * 8 + wi] = w;
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

// The same, one activation row per workgroup: the row is copied into LDS
// with 16-byte loads, then each thread writes eight consecutive outputs with
// one 16-byte store, gathering them from LDS. Memory sees contiguous reads
// and writes only. Needs K % 8 == 0, 16-byte aligned rows and 2K bytes of
// LDS.
__global__ __launch_bounds__(256) void q4_permute_rows_kernel(const uint16_t* __restrict__ x,
                                                              const int32_t* __restrict__ perm,
                                                              uint16_t* __restrict__ xp, int K)
{
    extern __shared__ q4dev::u4 row_lds[];
    uint16_t* row = reinterpret_cast<uint16_t*>(row_lds);
    const size_t base = (size_t)blockIdx.x * K;
    const int chunks = K >> 3;
    const q4dev::u4* src = reinterpret_cast<const q4dev::u4*>(x + base);
    for (int c = threadIdx.x; c < chunks; c += 256) row_lds[c] = src[c];
    __syncthreads();
    q4dev::u4* dst = reinterpret_cast<q4dev::u4*>(xp + base);
    const q4dev::u4* pv = reinterpret_cast<const q4dev::u4*>(perm);
    for (int c = threadIdx.x; c < chunks; c += 256) {
        const q4dev::u4 p0 = pv[2 * c], p1 = pv[2 * c + 1];
        q4dev::u4 o;
        o[0] = (uint32_t)row[p0[0]] | ((uint32_t)row[p0[1]] << 16);
        o[1] = (uint32_t)row[p0[2]] | ((uint32_t)row[p0[3]] << 16);
        o[2] = (uint32_t)row[p1[0]] | ((uint32_t)row[p1[1]] << 16);
        o[3] = (uint32_t)row[p1[2]] | ((uint32_t)row[p1[3]] << 16);
        dst[c] = o;
    }
}

// sz[g][n] = scale bits | zero point << 16, from the handle's scales and
// packed zeros (bits-wide codes, packed along N).
__global__ __launch_bounds__(256) void q4_make_sz_kernel(const uint16_t* __restrict__ scales,
                                                         const uint32_t* __restrict__ qzeros,
                                                         uint32_t* __restrict__ sz, int ng, int N, int bits)
{
    const size_t total = (size_t)ng * N;
    const int per = 32 / bits;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const size_t g = idx / N;
        const int n = (int)(idx % N);
        const uint32_t z = (qzeros[g * (N / per) + n / per] >> (bits * (n % per))) & ((1u << bits) - 1u);
        sz[idx] = (uint32_t)scales[idx] | (z << 16);
    }
}

// Debug dump: w[k][n] (original row order) = the dequantized weight (k, n) as
// each kernel forms it, rounded to fp16. FACTORED (skinny kernel): the
// kernel's own (q - z) from sub_zero_word times the fp32 scale, which is the
// exact weight the kernel applies, then one RNE rounding. Otherwise (GEMM):
// the fp16 value dequant_word feeds to the MFMA.
// BF: bfloat16 values of the bfloat16 forms -- FACTORED: the kernel's exact
// q - z as bfloat16 times the fp32 scale, rounded once to bfloat16;
// otherwise the bfloat16 weight mix_word feeds to the bfloat16 MFMA.
template <bool FACTORED, bool BF, bool W8>
__global__ __launch_bounds__(256) void q4_dump_kernel(const uint32_t* __restrict__ qweight,
                                                      const uint32_t* __restrict__ sz,
                                                      const int32_t* __restrict__ inv_perm,
                                                      uint16_t* __restrict__ w, int K, int N, int G)
{
    const size_t total = (size_t)K * N;
    for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * blockDim.x) {
        const int k = (int)(idx / N), n = (int)(idx % N);
        const int kk = inv_perm ? inv_perm[k] : k;       // sorted position of row k
        const int g = kk / G;
        int e;
        const size_t wp = private_word(kk, n, N, &e, W8 ? 8 : 4);
        // both kernels read the scale and the zero point from the group word
        const uint32_t z = sz[(size_t)g * N + n] >> 16;
        // the two words of the k-step (8-bit) or its one word (4-bit)
        const uint32_t word = qweight[wp];
        const uint32_t w0 = W8 ? qweight[wp - (e >> 2)] : word, w1 = W8 ? qweight[wp - (e >> 2) + 1] : word;
        const uint16_t sb = (uint16_t)sz[(size_t)g * N + n];
        if constexpr (BF) {
            float t = FACTORED ? 1.0f : f16_bits_to_f32(sb);
            asm("" : "+v"(t));    // as in the kernels: one fused multiply-add per value
            const b8 v = W8 ? mix_word8(w0, w1, mix_consts(z, t)) : mix_word(word, mix_consts(z, t));
            if (FACTORED)
                w[idx] = f32_to_bf16_bits(f16_bits_to_f32(sb) * static_cast<float>(v[e]));
            else
                w[idx] = bitcast<uint16_t>(v[e]);
        } else if (FACTORED) {
            const h8 d = W8 ? sub_zero_word8(w0, w1, zero_pair(z)) : sub_zero_word(word, zero_pair(z));
            w[idx] = f32_to_f16_bits(f16_bits_to_f32(sb) * static_cast<float>(d[e]));
        } else {
            const h8 v = W8 ? dequant_word8(w0, w1, zero_pair(z), scale_pair(sb))
                            : dequant_word(word, zero_pair(z), scale_pair(sb));
            w[idx] = bitcast<uint16_t>(v[e]);
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
                         int n_total, int col_off, int bits, hipStream_t stream)
{
    if (bits == 8)
        hipLaunchKernelGGL(q4_repack8_kernel, dim3(grid_for(packed_words(K, N, 8))), dim3(256), 0, stream,
                           src, perm, dst, K, N, n_total, col_off);
    else
        hipLaunchKernelGGL(q4_repack_kernel, dim3(grid_for(packed_words(K, N, 4))), dim3(256), 0, stream,
                           src, perm, dst, K, N, n_total, col_off);
    return hipGetLastError();
}

hipError_t launch_make_sz(q4_matrix* h, const uint16_t* scales, const uint32_t* qzeros, hipStream_t stream)
{
    hipLaunchKernelGGL(q4_make_sz_kernel, dim3(grid_for((size_t)h->ng * h->N)), dim3(256), 0, stream,
                       scales, qzeros, h->sz, h->ng, h->N, h->bits);
    return hipGetLastError();
}

hipError_t launch_permute_x(const uint16_t* x, const int32_t* perm, uint16_t* xp, int M, int K,
                            hipStream_t stream)
{
    // One workgroup per row has too little parallelism for a few rows (the
    // skinny kernel's M): those take the element-wise form. x rows are
    // 16-byte aligned when x is (K is a multiple of 8).
    constexpr int kMaxRowLds = 64 * 1024;
    if (M > Q4_GEMV_MAX_M && (size_t)K * 2 <= kMaxRowLds && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
        reinterpret_cast<uintptr_t>(xp) % 16 == 0 && reinterpret_cast<uintptr_t>(perm) % 16 == 0)
        hipLaunchKernelGGL(q4_permute_rows_kernel, dim3(M), dim3(256), (size_t)K * 2, stream, x, perm, xp, K);
    else
        hipLaunchKernelGGL(q4_permute_x_kernel, dim3(grid_for((size_t)M * K)), dim3(256), 0, stream, x,
                           perm, xp, M, K);
    return hipGetLastError();
}

template <bool W8>
hipError_t launch_dump_w(const q4_matrix* h, int path, uint16_t* w, bool bf16, hipStream_t stream)
{
    const dim3 grid(grid_for((size_t)h->K * h->N));
    const bool f = path == Q4_PATH_GEMV;
    if (f && bf16)
        hipLaunchKernelGGL((q4_dump_kernel<true, true, W8>), grid, dim3(256), 0, stream, h->qweight, h->sz,
                           h->inv_perm, w, h->K, h->N, h->G);
    else if (f)
        hipLaunchKernelGGL((q4_dump_kernel<true, false, W8>), grid, dim3(256), 0, stream, h->qweight, h->sz,
                           h->inv_perm, w, h->K, h->N, h->G);
    else if (bf16)
        hipLaunchKernelGGL((q4_dump_kernel<false, true, W8>), grid, dim3(256), 0, stream, h->qweight, h->sz,
                           h->inv_perm, w, h->K, h->N, h->G);
    else
        hipLaunchKernelGGL((q4_dump_kernel<false, false, W8>), grid, dim3(256), 0, stream, h->qweight, h->sz,
                           h->inv_perm, w, h->K, h->N, h->G);
    return hipGetLastError();
}

hipError_t launch_dump(const q4_matrix* h, int path, uint16_t* w, bool bf16, hipStream_t stream)
{
    return h->bits == 8 ? launch_dump_w<true>(h, path, w, bf16, stream)
                        : launch_dump_w<false>(h, path, w, bf16, stream);
}

}  // namespace q4
