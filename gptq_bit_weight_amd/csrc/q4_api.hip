// C ABI of libq4: handle construction, dispatch and debug entry points.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstring>
#include <map>
#include <utility>
#include <vector>

#include "q4_internal.h"

// The allocation-free entry point's workspace (q4_matmul_static): one copy
// per GPU. Host code never passes this name to a kernel or a copy; it uses
// the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[Q4_STATIC_SCRATCH_BYTES];

namespace q4 {

hipError_t launch_gemv(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
                       int M, int col_tiles, int splits, bool gather_x, bool bf16, float* partials,
                       uint32_t* counters, hipStream_t stream);
hipError_t launch_gemm_stream(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
                              int M, bool bf16, int waves, int workers, float* partials, uint32_t* counters,
                              hipStream_t stream);
hipError_t launch_repack(const uint32_t* src, const int32_t* perm, uint32_t* dst, int K, int N,
                         int n_total, int col_off, int bits, hipStream_t stream);
hipError_t launch_permute_x(const uint16_t* x, const int32_t* perm, uint16_t* xp, int M, int K,
                            hipStream_t stream);
hipError_t launch_dump(const q4_matrix* h, int path, uint16_t* w, bool bf16, hipStream_t stream);
hipError_t launch_make_sz(q4_matrix* h, const uint16_t* scales, const uint32_t* qzeros, hipStream_t stream);

namespace {

q4_status hip_fail(hipError_t e, const char* what)
{
    return fail(e == hipErrorOutOfMemory ? Q4_ERR_OOM : Q4_ERR_HIP, "%s: %s", what,
                hipGetErrorString(e));
}

#define Q4_HIP(call, what)                                  \
    do {                                                    \
        hipError_t e_ = (call);                             \
        if (e_ != hipSuccess) return hip_fail(e_, (what));  \
    } while (0)

void destroy(q4_matrix* h)
{
    if (!h) return;
    (void)hipFree(h->qweight);
    (void)hipFree(h->block);
    for (float* p : h->partials_grown) (void)hipFree(p);
    (void)hipFree(h->xperm);
    for (uint16_t* p : h->xperm_retired) (void)hipFree(p);
    delete h;
}

q4_status check_device(int* dev, int* num_cu)
{
    Q4_HIP(hipGetDevice(dev), "hipGetDevice");
    hipDeviceProp_t prop;
    Q4_HIP(hipGetDeviceProperties(&prop, *dev), "hipGetDeviceProperties");
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(Q4_ERR_DEVICE, "device %d is %s; libq4 is built for gfx950 (MI355X) only", *dev,
                    prop.gcnArchName);
    *num_cu = prop.multiProcessorCount;
    return Q4_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---- scratch of the allocation-free entry point (q4_matmul_static) -------
// One array per GPU, placed in device memory when q4_make first looks it up
// on that GPU and kept until the process ends: the first kStaticCounterBytes
// hold arrival counters (the
// skinny kernel's split-K or the GEMM's stream-K ones, which the kernels
// return to zero), then an act-order call's x[:, perm], then fp32 partial
// sums. Every q4_matmul_static call on a GPU uses that GPU's array, so calls
// that overlap in time on one GPU race.
constexpr size_t kStaticScratchBytes = (size_t)Q4_STATIC_SCRATCH_BYTES;
constexpr size_t kStaticCounterBytes = 64 << 10;
constexpr int kStaticCounters = (int)(kStaticCounterBytes / 4);

__global__ void q4_zero_words_kernel(uint32_t* p, int n)
{
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) p[i] = 0u;
}

std::mutex g_static_mutex;
auto* g_static = new std::map<int, unsigned char*>;   // device -> its copy of `scratch`

// Set-up of the static scratch on `device` (the current one), once per device
// and process, from q4_make (every handle is made on its device before any
// call uses it): look up this device's address of `scratch` (the HIP runtime
// places the array in device memory then) and clear its counters with a
// small kernel on the null stream, which q4_make's closing synchronization
// waits for. The kernels leave the counters at zero after every call.
q4_status static_setup(int device)
{
    std::lock_guard<std::mutex> lock(g_static_mutex);
    if (g_static->count(device)) return Q4_OK;
    void* ptr = nullptr;
    Q4_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "q4_make: static scratch address");
    if (!ptr) return fail(Q4_ERR_HIP, "q4_make: no device address for the static scratch array");
    hipLaunchKernelGGL(q4_zero_words_kernel, dim3((kStaticCounters + 255) / 256), dim3(256), 0, 0,
                       static_cast<uint32_t*>(ptr), kStaticCounters);
    Q4_HIP(hipGetLastError(), "q4_make: clear the static counters");
    (*g_static)[device] = static_cast<unsigned char*>(ptr);
    return Q4_OK;
}

// This device's copy of `scratch`, set up by q4_make.
q4_status static_scratch(int device, unsigned char** base)
{
    std::lock_guard<std::mutex> lock(g_static_mutex);
    auto it = g_static->find(device);
    if (it == g_static->end())
        return fail(Q4_ERR_INVALID_ARG, "q4_matmul_static: no handle was made on device %d", device);
    *base = it->second;
    return Q4_OK;
}

// One handle over the column concatenation of `parts` layers that share K,
// groupsize and g_idx (part i supplies columns [off_i, off_i + N[i]) of the
// result, in part order). q4_make is the one-part case.
q4_status make_impl(int parts, const int32_t* const* qweight, const int32_t* const* qzeros,
                    const uint16_t* const* scales, const int32_t* g_idx, int K, const int* Np,
                    int groupsize, int bits, const char* who, q4_matrix** out)
{
    if (bits != 4 && bits != 8) return fail(Q4_ERR_UNSUPPORTED, "%s: bits=%d is not 4 or 8", who, bits);
    if (parts < 1 || parts > kMaxParts)
        return fail(Q4_ERR_INVALID_ARG, "%s: parts=%d outside [1, %d]", who, parts, kMaxParts);
    if (!qweight || !scales || !Np)
        return fail(Q4_ERR_INVALID_ARG, "%s: null array argument", who);
    long long ntot = 0;
    for (int i = 0; i < parts; ++i) {
        if (!qweight[i] || !scales[i])
            return fail(Q4_ERR_INVALID_ARG, "%s: qweight and scales must be non-null (part %d)", who, i);
        if (Np[i] <= 0 || Np[i] % 8)
            return fail(Q4_ERR_INVALID_ARG, "%s: N=%d of part %d is not a positive multiple of 8", who, Np[i], i);
        if (!aligned(qweight[i], 16) || !aligned(scales[i], 8) || (qzeros && !aligned(qzeros[i], 4)))
            return fail(Q4_ERR_INVALID_ARG, "%s: qweight must be 16-byte aligned, scales 8-byte (part %d)",
                        who, i);
        ntot += Np[i];
    }
    if (ntot > INT_MAX) return fail(Q4_ERR_UNSUPPORTED, "%s: %lld columns in total", who, ntot);
    const int N = (int)ntot;
    int G = 0;
    q4_status st = check_shape(K, N, groupsize, &G, bits);
    if (st != Q4_OK) return st;
    int dev = -1, num_cu = 0;
    st = check_device(&dev, &num_cu);
    if (st != Q4_OK) return st;
    // The inputs may still be being written by work on other streams.
    Q4_HIP(hipDeviceSynchronize(), "q4_make: synchronize");
    st = static_setup(dev);
    if (st != Q4_OK) return st;

    const int ng = K / G;
    std::vector<int32_t> perm;
    int act = 0;
    if (g_idx) {
        std::vector<int32_t> gh(K);
        Q4_HIP(hipMemcpy(gh.data(), g_idx, sizeof(int32_t) * K, hipMemcpyDeviceToHost),
               "q4_make: copy g_idx");
        perm.resize(K);
        int trivial = 0;
        st = plan_actorder(gh.data(), K, G, perm.data(), &trivial);
        if (st != Q4_OK) return st;
        act = trivial ? 0 : 1;
    }

    q4_matrix* h = new q4_matrix();
    h->K = K;
    h->N = N;
    h->G = G;
    h->ng = ng;
    h->act_order = act;
    h->bits = bits;
    h->device = dev;
    h->num_cu = num_cu;
    auto bail = [&](q4_status s) {
        destroy(h);
        return s;
    };
    hipError_t e;
    // Split-K partials for the largest splits x M the plan takes at any M
    // the automatic dispatch gives the skinny kernel (none for most layers).
    int max_rows = 0;
    for (int m = 1; m <= kGemvMaxM; ++m) {
        if (!gemv_serves(m, K, N, G, bits)) continue;
        int ct = 0, sp = 0;
        plan_gemv(m, K, N, G, num_cu, &ct, &sp, bits);
        if (sp > 1) max_rows = std::max(max_rows, sp * m);
    }
    // The handle keeps two device allocations: the packed weights, and one
    // carved into 256-byte aligned regions for everything else (the device
    // allocator rounds large allocations up to 2 MiB, so the small buffers
    // share one instead of each being rounded on its own).
    const int col_tiles = (N + 15) / 16;
    const bool staged = act && num_kblocks(K) * kBlockK <= kGemvXRows;
    size_t offs[6], total = 0;
    const size_t sizes[6] = {(size_t)ng * N * 4, (size_t)col_tiles * 4, act ? (size_t)K * 4 : 0,
                             act ? (size_t)K * 4 : 0, staged ? (size_t)K * 2 : 0, (size_t)max_rows * N * 4};
    for (int r = 0; r < 6; ++r) {
        offs[r] = total;
        total += (sizes[r] + 255) & ~(size_t)255;
    }
    if ((e = hipMalloc(&h->qweight, packed_words(K, N, bits) * 4)) != hipSuccess)
        return bail(hip_fail(e, "q4_make: qweight"));
    if ((e = hipMalloc(&h->block, total)) != hipSuccess) return bail(hip_fail(e, "q4_make: device memory"));
    h->block_bytes = total;
    char* base = static_cast<char*>(h->block);
    h->sz = reinterpret_cast<uint32_t*>(base + offs[0]);
    h->counters = reinterpret_cast<uint32_t*>(base + offs[1]);
    if (act) {
        h->perm = reinterpret_cast<int32_t*>(base + offs[2]);
        h->inv_perm = reinterpret_cast<int32_t*>(base + offs[3]);
    }
    if (staged) h->inv16 = reinterpret_cast<uint16_t*>(base + offs[4]);
    if (max_rows > 0) {
        h->partials = reinterpret_cast<float*>(base + offs[5]);
        h->partial_rows = max_rows;
    }
    if ((e = hipMemset(h->counters, 0, (size_t)col_tiles * 4)) != hipSuccess) return bail(hip_fail(e, "q4_make: counters"));
    if (act) {
        std::vector<int32_t> inv(K);
        for (int k = 0; k < K; ++k) inv[perm[k]] = k;
        if ((e = hipMemcpy(h->perm, perm.data(), (size_t)K * 4, hipMemcpyHostToDevice)) != hipSuccess)
            return bail(hip_fail(e, "q4_make: perm"));
        if ((e = hipMemcpy(h->inv_perm, inv.data(), (size_t)K * 4, hipMemcpyHostToDevice)) != hipSuccess)
            return bail(hip_fail(e, "q4_make: perm"));
        // 16-bit copy for the skinny kernel's own activation staging, which
        // takes layers of at most kGemvXRows rows
        if (staged) {
            std::vector<uint16_t> inv16(inv.begin(), inv.end());
            if ((e = hipMemcpy(h->inv16, inv16.data(), (size_t)K * 2, hipMemcpyHostToDevice)) != hipSuccess)
                return bail(hip_fail(e, "q4_make: perm"));
        }
    }
    // The checkpoint's scales and packed zeros, gathered with the handle's
    // row pitch into temporaries from which the group words are built. Part
    // i's scales and zero words are columns off_i .. off_i + N_i of the
    // rows (zero words: off_i / 8 .., every offset a multiple of 8).
    uint16_t* tscales = nullptr;
    uint32_t* tqzeros = nullptr;
    auto bail_tmp = [&](q4_status st) {
        (void)hipDeviceSynchronize();
        (void)hipFree(tscales);
        (void)hipFree(tqzeros);
        return bail(st);
    };
    const size_t zrow = (size_t)N * bits / 8;   // bytes per row of packed zeros
    if ((e = hipMalloc(&tscales, (size_t)ng * N * 2)) != hipSuccess) return bail_tmp(hip_fail(e, "q4_make: scales"));
    if ((e = hipMalloc(&tqzeros, (size_t)ng * zrow)) != hipSuccess) return bail_tmp(hip_fail(e, "q4_make: qzeros"));
    int off = 0;
    for (int i = 0; i < parts; ++i) {
        if ((e = hipMemcpy2D(tscales + off, (size_t)N * 2, scales[i], (size_t)Np[i] * 2, (size_t)Np[i] * 2,
                             (size_t)ng, hipMemcpyDeviceToDevice)) != hipSuccess)
            return bail_tmp(hip_fail(e, "q4_make: scales"));
        // A part without zeros is symmetric: every zero point is
        // 2^(bits-1) (GPTQModel wiki "Inference Backends", section
        // "Packing, conversion, and runtime initialization", row "Missing
        // zeros"): 8, zero words 0x88888888, or 128, zero bytes 0x80. The
        // part's zeros occupy bytes off * bits / 8 .. of each row (off and
        // N[i] are multiples of 8, so no word is shared between parts).
        const int32_t* qz = qzeros ? qzeros[i] : nullptr;
        char* zdst = reinterpret_cast<char*>(tqzeros) + (size_t)off * bits / 8;
        const size_t zpart = (size_t)Np[i] * bits / 8;
        if (qz)
            e = hipMemcpy2D(zdst, zrow, qz, zpart, zpart, (size_t)ng, hipMemcpyDeviceToDevice);
        else
            e = hipMemset2D(zdst, zrow, bits == 8 ? 0x80 : 0x88, zpart, (size_t)ng);
        if (e != hipSuccess) return bail_tmp(hip_fail(e, "q4_make: qzeros"));
        if ((e = launch_repack(reinterpret_cast<const uint32_t*>(qweight[i]), h->perm, h->qweight, K, Np[i], N,
                               off, bits, 0)) != hipSuccess)
            return bail_tmp(hip_fail(e, "q4_make: repack launch"));
        off += Np[i];
    }
    if ((e = launch_make_sz(h, tscales, tqzeros, 0)) != hipSuccess)
        return bail_tmp(hip_fail(e, "q4_make: group parameters"));
    if ((e = hipDeviceSynchronize()) != hipSuccess) return bail_tmp(hip_fail(e, "q4_make: repack"));
    (void)hipFree(tscales);
    (void)hipFree(tqzeros);
    *out = h;
    return Q4_OK;
}

int choose_path(const q4_matrix* h, int M, int forced)
{
    if (M == 0) return Q4_PATH_NONE;
    if (forced == Q4_PATH_MFMA) return Q4_PATH_MFMA;
    if (forced == Q4_PATH_GEMV) return M <= kGemvMaxM ? Q4_PATH_GEMV : -1;
    return gemv_serves(M, h->K, h->N, h->G, h->bits) ? Q4_PATH_GEMV : Q4_PATH_MFMA;
}

// Grow the act-order activation workspace to hold M x K halfs.
q4_status ensure_xperm(const q4_matrix* h, int M, hipStream_t stream)
{
    const size_t need = (size_t)M * h->K;
    std::lock_guard<std::mutex> lock(h->ws_mutex);
    if (h->xperm_elems >= need) return Q4_OK;
    // Growing allocates, which a stream under graph capture cannot do: say
    // so instead of breaking the capture.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    Q4_HIP(hipStreamIsCapturing(stream, &cap), "q4_matmul: capture query");
    if (cap != hipStreamCaptureStatusNone)
        return fail(Q4_ERR_INVALID_ARG,
                    "q4_matmul: the act-order workspace must grow to M=%d under stream capture; "
                    "make one uncaptured call with this M (or larger) first", M);
    // Earlier launches, and graphs captured from them, may still use the old
    // buffer: retire it (freed with the handle) instead of freeing it now.
    uint16_t* fresh = nullptr;
    Q4_HIP(hipMalloc(&fresh, need * 2), "q4_matmul: act-order workspace");
    if (h->xperm) h->xperm_retired.push_back(h->xperm);
    h->xperm = fresh;
    h->xperm_elems = need;
    return Q4_OK;
}

// Grow the skinny kernel's split-K partials to hold splits x M rows (an
// explicit split count, or explicit skinny-kernel M, above the planned ones).
q4_status ensure_partials(const q4_matrix* h, int splits, int M, hipStream_t stream)
{
    std::lock_guard<std::mutex> lock(h->ws_mutex);
    const int rows = splits * M;
    if (h->partial_rows >= rows) return Q4_OK;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    Q4_HIP(hipStreamIsCapturing(stream, &cap), "q4_matmul: capture query");
    if (cap != hipStreamCaptureStatusNone)
        return fail(Q4_ERR_INVALID_ARG,
                    "q4_matmul: the split-K workspace must grow to %d splits of %d rows under stream "
                    "capture; make one uncaptured call with this split count and M first", splits, M);
    float* fresh = nullptr;
    Q4_HIP(hipMalloc(&fresh, (size_t)rows * h->N * 4), "q4_matmul: split-K workspace");
    // earlier launches (and graphs captured from them) may still use the old
    // buffer: it stays allocated until the handle is freed
    h->partials_grown.push_back(fresh);
    h->partials = fresh;
    h->partial_rows = rows;
    return Q4_OK;
}

// Stream-K workspace of the streaming GEMM, one per (device, stream): two
// fp32 slots of one output tile and one arrival counter per workgroup. The
// first one holds two 256 x 128 slots for each of max(workers, 2 x CUs)
// workgroups rounded up to a power of two (128 MiB on 256 CUs, which is also
// two 256 x 256 slots for each of 256 eight-wave workgroups); it is doubled
// until a call fits. Calls on one stream run in order, so they can share it whatever
// handle they use; calls on different streams get different buffers. A
// workspace that is outgrown is replaced but never freed (a captured graph
// may still name it); all are kept until the process ends.
struct SkSpace {
    float* partials = nullptr;
    uint32_t* counters = nullptr;
    size_t partial_bytes = 0;   // capacity of partials
    int counter_count = 0;      // capacity of counters (one per workgroup)
};
std::mutex g_sk_mutex;
auto* g_sk = new std::map<std::pair<int, hipStream_t>, SkSpace>;

// Fills *ws for `workers` workgroups with partial-sum slots of slot_bytes
// (two per workgroup) on (device, stream). Under stream capture a missing or
// small workspace cannot be allocated: *ws is then left empty.
q4_status sk_workspace(int device, int num_cu, hipStream_t stream, int workers, size_t slot_bytes, SkSpace* ws)
{
    std::lock_guard<std::mutex> lock(g_sk_mutex);
    SkSpace& sp = (*g_sk)[{device, stream}];
    if (sp.partial_bytes >= 2 * (size_t)workers * slot_bytes && sp.counter_count >= workers) {
        *ws = sp;
        return Q4_OK;
    }
    *ws = SkSpace{};
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    Q4_HIP(hipStreamIsCapturing(stream, &cap), "q4_matmul: capture query");
    if (cap != hipStreamCaptureStatusNone) return Q4_OK;
    // at least two 256 x 128 slots for each of 2 num_cu workgroups (what any
    // planned call needs), doubled until this call fits
    int n = 2 * std::max(num_cu, 1);
    while (n < workers) n *= 2;
    size_t bytes = 2 * (size_t)n * kGemmBM * kGemmBN * sizeof(float);
    while (bytes < 2 * (size_t)workers * slot_bytes) bytes *= 2;
    SkSpace fresh;
    Q4_HIP(hipMalloc(&fresh.partials, bytes), "q4_matmul: stream-K partials");
    if (hipMalloc(&fresh.counters, (size_t)n * sizeof(uint32_t)) != hipSuccess) {
        (void)hipFree(fresh.partials);
        return fail(Q4_ERR_OOM, "q4_matmul: stream-K counters");
    }
    Q4_HIP(hipMemsetAsync(fresh.counters, 0, (size_t)n * sizeof(uint32_t), stream),
           "q4_matmul: stream-K counters");
    fresh.partial_bytes = bytes;
    fresh.counter_count = n;
    sp = fresh;
    *ws = sp;
    return Q4_OK;
}

// The handle's buffers live on the device it was made on, which must be
// the current one (kernels run on the current device).
q4_status check_current(const q4_matrix* h, const char* who)
{
    int cur = -1;
    Q4_HIP(hipGetDevice(&cur), "hipGetDevice");
    if (cur != h->device)
        return fail(Q4_ERR_INVALID_ARG, "%s: the handle was made on device %d, the current device is %d", who,
                    h->device, cur);
    return Q4_OK;
}

// `stat`: q4_matmul_static (every workspace from the device's scratch
// array, nothing allocated); otherwise workspaces are the handle's and the
// stream's, allocated or grown on demand.
q4_status matmul_impl(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
                      int M, int path, int variant, int splits, bool bf16, hipStream_t stream,
                      bool stat = false)
{
    if (!h) return fail(Q4_ERR_INVALID_ARG, "q4_matmul: null handle");
    if (q4_status st = check_current(h, "q4_matmul"); st != Q4_OK) return st;
    if (M < 0) return fail(Q4_ERR_INVALID_ARG, "q4_matmul: M=%d is negative", M);
    if (M == 0) return Q4_OK;
    if (!x || !out) return fail(Q4_ERR_INVALID_ARG, "q4_matmul: x and out must be non-null");
    if (!aligned(x, 16)) return fail(Q4_ERR_INVALID_ARG, "q4_matmul: x must be 16-byte aligned");
    // Byte offsets inside x stay below 2^31 (out-of-range lanes add 2^31).
    if ((long long)M * h->K * 2 > INT_MAX || (long long)M * h->N > INT_MAX)
        return fail(Q4_ERR_UNSUPPORTED, "q4_matmul: M=%d too large for this layer (M*K*2 must be < 2^31)", M);
    {
        const char* xb = reinterpret_cast<const char*>(x);
        const char* ob = reinterpret_cast<const char*>(out);
        const size_t xs = (size_t)M * h->K * 2, os = (size_t)M * h->N * 2;
        if (xb < ob + os && ob < xb + xs) return fail(Q4_ERR_INVALID_ARG, "q4_matmul: out overlaps x");
    }
    const int kind = choose_path(h, M, path);
    if (kind < 0)
        return fail(Q4_ERR_INVALID_ARG, "q4_matmul: the skinny kernel takes M <= %d (M=%d)",
                    kGemvMaxM, M);
    if (kind == Q4_PATH_GEMV) {
        if (splits < 0 || splits > kMaxSplits)
            return fail(Q4_ERR_INVALID_ARG, "q4_matmul: splits=%d outside [0, %d]", splits, kMaxSplits);
        if (variant != 0 && variant != 1 && variant != 2 && variant != 4)
            return fail(Q4_ERR_INVALID_ARG, "q4_matmul: skinny-kernel tiles %d not 0, 1, 2 or 4", variant);
        if (h->bits == 8 && variant == 4)
            return fail(Q4_ERR_UNSUPPORTED, "q4_matmul: 8-bit weights take at most 2 column tiles");
    } else {
        if (variant != 0 && variant != 3 && variant != 4 && variant != 8)
            return fail(Q4_ERR_INVALID_ARG, "q4_matmul: GEMM variant %d is not 0, 3, 4 or 8", variant);
        if (variant == 8 && gemm_bm(M) != kGemmBM)
            return fail(Q4_ERR_INVALID_ARG, "q4_matmul: 256-column GEMM tiles (variant 8) need M > %d (M=%d)",
                        kGemmSmallM, M);
        if (splits < 0 || splits > Q4_GEMM_MAX_WORKERS)
            return fail(Q4_ERR_INVALID_ARG, "q4_matmul: GEMM workgroups %d outside [0, %d]", splits,
                        Q4_GEMM_MAX_WORKERS);
    }

    int ct = 0, s = 0;
    bool gather = false;
    if (kind == Q4_PATH_GEMV) {
        plan_gemv(M, h->K, h->N, h->G, h->num_cu, &ct, &s, h->bits);
        if (variant) ct = variant;
        if (splits) s = splits;
        // act-order: without K splits, the skinny kernel stages x[:, perm]
        // in LDS itself when all of it fits
        gather = h->act_order && h->inv16 && gemv_gathers_x(M, h->K, s);
    }
    // Static scratch: [counters | x[:, perm] (act-order without staging) |
    // fp32 partials]. The sizes are fixed before anything is launched.
    unsigned char* base = nullptr;
    size_t xp_bytes = 0, part_bytes = 0;
    if (stat) {
        if (h->act_order && !gather) {
            xp_bytes = ((size_t)M * h->K * 2 + 255) & ~(size_t)255;
            if (xp_bytes > kStaticScratchBytes - kStaticCounterBytes)
                return fail(Q4_ERR_UNSUPPORTED,
                            "q4_matmul_static: the act-order activations (M*K*2 = %zu bytes) exceed the "
                            "%zu-byte static workspace; use q4_matmul_bias",
                            (size_t)M * h->K * 2, kStaticScratchBytes - kStaticCounterBytes);
        }
        part_bytes = kStaticScratchBytes - kStaticCounterBytes - xp_bytes;
        if (kind == Q4_PATH_GEMV) {
            // fewer K splits when their partials or counters do not fit (the
            // plan's counts are powers of two)
            while (s > 1 && ((size_t)s * M * h->N * 4 > part_bytes || (h->N + 15) / 16 > kStaticCounters)) s /= 2;
            gather = h->act_order && h->inv16 && gemv_gathers_x(M, h->K, s);
            if (h->act_order && !gather && xp_bytes == 0)
                return fail(Q4_ERR_UNSUPPORTED, "q4_matmul_static: no room for the act-order activations");
        }
        q4_status st = static_scratch(h->device, &base);
        if (st != Q4_OK) return st;
    }
    const uint16_t* xe = x;
    if (h->act_order && !gather) {
        uint16_t* xp = nullptr;
        if (stat) {
            xp = reinterpret_cast<uint16_t*>(base + kStaticCounterBytes);
        } else {
            q4_status st = ensure_xperm(h, M, stream);
            if (st != Q4_OK) return st;
            xp = h->xperm;
        }
        Q4_HIP(launch_permute_x(x, h->perm, xp, M, h->K, stream), "q4_matmul: permute launch");
        xe = xp;
    }
    if (kind == Q4_PATH_GEMV) {
        float* partials = h->partials;
        uint32_t* counters = h->counters;
        if (stat) {
            partials = reinterpret_cast<float*>(base + kStaticCounterBytes + xp_bytes);
            counters = reinterpret_cast<uint32_t*>(base);
        } else if (s > 1) {
            q4_status st = ensure_partials(h, s, M, stream);
            if (st != Q4_OK) return st;
            partials = h->partials;
        }
        Q4_HIP(launch_gemv(h, xe, bias, out, M, ct, s, gather, bf16, partials, counters, stream),
               "q4_matmul: gemv launch");
    } else {
        // splits: 0 planned, 1 one workgroup per output tile, P >= 2
        // workgroups sharing the tiles' k-iterations (stream-K)
        // (the GEMM's work split is 32-bit arithmetic; the narrow tiles are
        // the more numerous)
        if ((long long)gemm_tiles(M, h->N, 4) * ((h->K + kGemmBK - 1) / kGemmBK) >= (1LL << 30))
            return fail(Q4_ERR_UNSUPPORTED, "q4_matmul: M=%d gives more than 2^30 GEMM (tile, k-step) pairs", M);
        // tile width: planned (variant 0 or 3) or explicit
        const int waves = variant == 4 || variant == 8 ? variant : gemm_waves(M, h->N, h->K, h->num_cu, h->bits);
        const int tiles = gemm_tiles(M, h->N, waves);
        int workers = splits == 0 ? plan_gemm_workers(M, h->N, h->K, h->num_cu, waves) : splits == 1 ? tiles : splits;
        // every workgroup must get at least one (tile, k-step) iteration:
        // a split tile counts its contributors as a range of workgroups
        workers = (int)std::min<long long>(workers, (long long)tiles * ((h->K + kGemmBK - 1) / kGemmBK));
        SkSpace ws;
        if (stat && workers != tiles) {
            // as many stream-K workgroups as the plan asks for and the
            // partials region holds (two slots of bm x (32 waves) fp32 each),
            // else one workgroup per tile
            const size_t per_worker = 2 * (size_t)gemm_bm(M) * (32 * waves) * sizeof(float);
            workers = (int)std::min<size_t>((size_t)workers, part_bytes / per_worker);
            workers = std::min(workers, kStaticCounters);
            if (workers < 2) workers = tiles;
            ws.partials = reinterpret_cast<float*>(base + kStaticCounterBytes + xp_bytes);
            ws.counters = reinterpret_cast<uint32_t*>(base);
        } else if (workers != tiles) {
            q4_status st = sk_workspace(h->device, h->num_cu, stream, workers,
                                        (size_t)gemm_bm(M) * (32 * waves) * sizeof(float), &ws);
            if (st != Q4_OK) return st;
            if (!ws.partials) {
                if (splits != 0)
                    return fail(Q4_ERR_INVALID_ARG,
                                "q4_matmul: the stream-K workspace for %d workgroups must be made "
                                "under no stream capture; make one uncaptured call first", workers);
                workers = tiles;   // planned call under capture: one workgroup per tile
            }
        }
        Q4_HIP(launch_gemm_stream(h, xe, bias, out, M, bf16, waves, workers, ws.partials, ws.counters, stream),
               "q4_matmul: gemm launch");
    }
    return Q4_OK;
}

}  // namespace
}  // namespace q4

extern "C" {

q4_matrix* q4_make(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                   const int32_t* g_idx, int K, int N, int groupsize)
{
    q4_matrix* h = nullptr;
    return q4::make_impl(1, &qweight, &qzeros, &scales, g_idx, K, &N, groupsize, 4, "q4_make", &h) == Q4_OK
               ? h
               : nullptr;
}

q4_matrix* q4_make_bits(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                        const int32_t* g_idx, int K, int N, int groupsize, int bits)
{
    q4_matrix* h = nullptr;
    return q4::make_impl(1, &qweight, &qzeros, &scales, g_idx, K, &N, groupsize, bits, "q4_make_bits",
                         &h) == Q4_OK
               ? h
               : nullptr;
}

q4_matrix* q4_make_cat(int parts, const int32_t* const* qweight, const int32_t* const* qzeros,
                       const uint16_t* const* scales, const int32_t* g_idx, int K, const int* N,
                       int groupsize)
{
    q4_matrix* h = nullptr;
    return q4::make_impl(parts, qweight, qzeros, scales, g_idx, K, N, groupsize, 4, "q4_make_cat", &h) == Q4_OK
               ? h
               : nullptr;
}

q4_matrix* q4_make_cat_bits(int parts, const int32_t* const* qweight, const int32_t* const* qzeros,
                            const uint16_t* const* scales, const int32_t* g_idx, int K, const int* N,
                            int groupsize, int bits)
{
    q4_matrix* h = nullptr;
    return q4::make_impl(parts, qweight, qzeros, scales, g_idx, K, N, groupsize, bits, "q4_make_cat_bits",
                         &h) == Q4_OK
               ? h
               : nullptr;
}

q4_status q4_matmul(const q4_matrix* h, const uint16_t* x, uint16_t* out, int M, hipStream_t stream)
{
    return q4::matmul_impl(h, x, nullptr, out, M, 0, 0, 0, false, stream);
}

q4_status q4_matmul_bias(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
                         int M, hipStream_t stream)
{
    return q4::matmul_impl(h, x, bias, out, M, 0, 0, 0, false, stream);
}

q4_status q4_matmul_ex(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
                       int M, int path, int variant, int splits, hipStream_t stream)
{
    if (path != 0 && path != Q4_PATH_GEMV && path != Q4_PATH_MFMA)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_matmul_ex: unknown path %d", path);
    return q4::matmul_impl(h, x, bias, out, M, path, variant, splits, false, stream);
}

q4_status q4_matmul_static(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
                           int M, hipStream_t stream)
{
    return q4::matmul_impl(h, x, bias, out, M, 0, 0, 0, false, stream, true);
}

q4_status q4_matmul_bf16(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
                         int M, hipStream_t stream)
{
    return q4::matmul_impl(h, x, bias, out, M, 0, 0, 0, true, stream);
}

q4_status q4_matmul_ex_bf16(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
                            int M, int path, int variant, int splits, hipStream_t stream)
{
    if (path != 0 && path != Q4_PATH_GEMV && path != Q4_PATH_MFMA)
        return q4::fail(Q4_ERR_INVALID_ARG, "q4_matmul_ex_bf16: unknown path %d", path);
    return q4::matmul_impl(h, x, bias, out, M, path, variant, splits, true, stream);
}

void q4_free(q4_matrix* h) { q4::destroy(h); }

int q4_path_for(const q4_matrix* h, int M)
{
    if (!h || M < 0) return -1;
    return q4::choose_path(h, M, 0);
}

int q4_gemv_gather(const q4_matrix* h, int M, int splits)
{
    if (!h || M < 1 || M > q4::kGemvMaxM || splits < 0 || splits > q4::kMaxSplits) return -1;
    if (!h->act_order || !h->inv16) return 0;
    int ct = 0, s = 0;
    q4::plan_gemv(M, h->K, h->N, h->G, h->num_cu, &ct, &s, h->bits);
    return q4::gemv_gathers_x(M, h->K, splits ? splits : s) ? 1 : 0;
}

int q4_handle_bits(const q4_matrix* h) { return h ? h->bits : -1; }

int q4_handle_info(const q4_matrix* h, int* K, int* N, int* groupsize, int* act_order)
{
    if (!h) return -1;
    if (K) *K = h->K;
    if (N) *N = h->N;
    if (groupsize) *groupsize = h->G;
    if (act_order) *act_order = h->act_order;
    return 0;
}

static q4_status dump_impl(const q4_matrix* h, int path, uint16_t* w, bool bf16, hipStream_t stream,
                           const char* who)
{
    if (!h || !w) return q4::fail(Q4_ERR_INVALID_ARG, "%s: null argument", who);
    if (q4_status st = q4::check_current(h, who); st != Q4_OK) return st;
    if (path != Q4_PATH_GEMV && path != Q4_PATH_MFMA)
        return q4::fail(Q4_ERR_INVALID_ARG, "%s: unknown path %d", who, path);
    hipError_t e = q4::launch_dump(h, path, w, bf16, stream);
    if (e != hipSuccess) return q4::fail(Q4_ERR_HIP, "%s: %s", who, hipGetErrorString(e));
    return Q4_OK;
}

q4_status q4_dequant_dump(const q4_matrix* h, int path, uint16_t* w, hipStream_t stream)
{
    return dump_impl(h, path, w, false, stream, "q4_dequant_dump");
}

q4_status q4_dequant_dump_bf16(const q4_matrix* h, int path, uint16_t* w, hipStream_t stream)
{
    return dump_impl(h, path, w, true, stream, "q4_dequant_dump_bf16");
}

}  // extern "C"
