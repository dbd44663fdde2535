// Read-bandwidth probe: the rate at which this GPU streams a buffer of a given
// size from HBM with the skinny kernel's kind of load (16 bytes a lane,
// non-temporal), with no arithmetic besides folding the words together. A
// measurement helper, not part of the product: it gives the achievable read
// rate of one launch of a given size, against which the fused kernels'
// effective bandwidth is compared.
#include <hip/hip_runtime.h>

#include "q4_internal.h"

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kLoads = 4;                         // 16-byte loads per lane per chunk
constexpr int kChunk = kThreads * kLoads;         // 16-byte words per chunk (16 KiB)

// Chunk c (16 KiB) is read by workgroup c % gridDim.x; lane t of it reads
// words t, t + 256, t + 512, t + 768. The folded words are stored only when
// they match a constant, so the loads cannot be dropped and nothing is
// written in practice.
__global__ __launch_bounds__(kThreads) void q4_read_probe_kernel(const u4* __restrict__ p, size_t chunks,
                                                                 uint32_t* __restrict__ sink)
{
    uint32_t acc = 0;
    for (size_t c = blockIdx.x; c < chunks; c += gridDim.x) {
        const u4* q = p + c * kChunk + threadIdx.x;
        u4 v[kLoads];
#pragma unroll
        for (int i = 0; i < kLoads; ++i) v[i] = __builtin_nontemporal_load(q + i * kThreads);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x & 255] = acc;
}

}  // namespace

extern "C" q4_status q4_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream)
{
    constexpr size_t chunk_bytes = (size_t)kChunk * 16;
    if (!buf || !sink) return q4::fail(Q4_ERR_INVALID_ARG, "q4_read_probe: null pointer");
    if (reinterpret_cast<uintptr_t>(buf) % 16)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_read_probe: buf must be 16-byte aligned");
    if (bytes == 0 || bytes % chunk_bytes)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_read_probe: bytes=%zu is not a positive multiple of %zu",
                        bytes, chunk_bytes);
    const size_t chunks = bytes / chunk_bytes;
    // Up to eight workgroups per CU of a 256-CU chip; small buffers get one
    // workgroup per chunk.
    const unsigned grid = (unsigned)(chunks < 2048 ? chunks : 2048);
    hipLaunchKernelGGL(q4_read_probe_kernel, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const u4*>(buf), chunks, sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return q4::fail(Q4_ERR_HIP, "q4_read_probe: %s", hipGetErrorString(e));
    return Q4_OK;
}
