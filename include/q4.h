/*
 * q4.h -- C ABI of libq4: the fused GPTQ 4-bit dequantize-and-multiply on
 * AMD Instinct MI355X (gfx950).
 *
 *   y[m,n] = sum_k x[m,k] * W[k,n],  W[k,n] = s[g(k),n] * (q[k,n] - z[g(k),n])
 *
 * The packed 4-bit weights are read from device memory and unpacked and
 * dequantized in registers; no dequantized weight matrix is ever written to
 * memory ("GPTQ's 'Exllama Kernel Not Installed' Warning", section "What the
 * fallback actually does"). The interface follows the handle + matmul pair of
 * "Implementation: Predibase Lorax GPTQ Exllama V1" (Description: a handle is
 * made once from qweight, qzeros, scales and an optional g_idx; the matmul
 * takes a 2-D activation and produces (batch, width)).
 *
 * Conventions for every entry point:
 *  - All tensor pointers passed to q4_make / q4_matmul* / q4_dequant_dump are
 *    DEVICE pointers on the current HIP device, to dense row-major data. A
 *    handle is used on the device it was made on: q4_matmul* and
 *    q4_dequant_dump return Q4_ERR_INVALID_ARG when another device is
 *    current.
 *  - fp16 data is passed as uint16_t bit patterns (IEEE binary16).
 *  - A failing call returns NULL or a non-zero q4_status, enqueues nothing and
 *    leaves every output untouched; q4_last_error() then holds the reason
 *    (thread-local, valid until the next failing call on that thread).
 *  - There is no silent fallback: when a case is not implemented on the GPU
 *    the call fails with Q4_ERR_UNSUPPORTED.
 *  - Calls that take a stream enqueue work on it and return without waiting;
 *    faults inside a kernel surface at the caller's next synchronization.
 *
 * Tensor formats (GPTQ checkpoint layout; "GPTQ's 'Exllama Kernel Not
 * Installed' Warning", section "Why the kernel is missing": 32-bit words
 * carrying 4-bit codes, a scale and a zero point for each group; I/O
 * contract table of the Lorax page: qweight/qzeros int32, scales fp16, g_idx
 * int32 or absent, bits = 4):
 *  - qweight int32 [K/8][N]: word (r, n) holds the codes of input rows
 *    k = 8r .. 8r+7 of column n, the code of k = 8r+i in bits 4i .. 4i+3.
 *  - qzeros  int32 [ceil(K/G)][N/8]: word (g, c) holds the zero points of
 *    columns n = 8c .. 8c+7 of group g, in the same nibble order. The stored
 *    nibble is the zero point itself (no offset).
 *  - scales  fp16  [ceil(K/G)][N].
 *  - g_idx   int32 [K] or NULL: group of input row k. NULL means g(k) = k / G.
 *  - x fp16 [M][K], out fp16 [M][N], bias fp16 [N].
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct q4_matrix q4_matrix;   /* opaque handle, immutable after q4_make */

typedef enum {
    Q4_OK = 0,
    Q4_ERR_INVALID_ARG = 1,   /* null pointer, bad shape or value            */
    Q4_ERR_UNSUPPORTED = 2,   /* valid input the GPU path does not implement */
    Q4_ERR_DEVICE = 3,        /* current device is not gfx950                */
    Q4_ERR_HIP = 4,           /* a HIP runtime call failed                   */
    Q4_ERR_OOM = 5            /* device allocation failed                    */
} q4_status;

/* Kernel identifiers returned by q4_path_for / accepted by q4_dequant_dump. */
enum {
    Q4_PATH_NONE = 0,   /* M == 0: nothing is launched                            */
    Q4_PATH_GEMV = 1,   /* bandwidth-bound skinny kernel, 1 <= M <= Q4_GEMV_MAX_M */
    Q4_PATH_MFMA = 2    /* LDS-staged MFMA GEMM for larger M                      */
};

/* Most rows the skinny kernel takes: q4_matmul runs it for 1 <= M <= 32 and
 * the MFMA GEMM above (q4_path_for tells which). */
#define Q4_GEMV_MAX_M 32
/* Most workgroups one streaming-GEMM launch may be given (q4_matmul_ex). */
#define Q4_GEMM_MAX_WORKERS 1024

/*
 * q4_make -- build a handle from GPTQ tensors (Lorax page, Description: the
 * handle is made once from the packed weights, zero points, scales and an
 * optional group index, and act-order is recognised from a g_idx that is not
 * the identity grouping).
 *
 * Arguments: device pointers qweight and scales (required), qzeros (NULL for
 * a symmetric layer stored without zeros: every zero point is then
 * 2^(bits-1) = 8, as GPTQModel wiki "Inference Backends", section "Packing,
 * conversion, and runtime initialization", row "Missing zeros" synthesizes
 * it), g_idx (optional, NULL allowed); K, N > 0 with K % 32 == 0 and
 * N % 8 == 0;
 * groupsize in {32, 64, 128, 256} with K % groupsize == 0, or -1 for one
 * group spanning K (then K % 32 == 0 still applies).
 *
 * Act-order: a g_idx equal to k / groupsize for every k is trivial and is
 * dropped (same result bit for bit as NULL). Otherwise the rows are reordered
 * by one stable argsort of g_idx (GPTQModel wiki "Inference Backends",
 * section "Runtime cache lifetime"); the sorted g_idx must equal
 * k / groupsize (every group exactly groupsize rows), else
 * Q4_ERR_UNSUPPORTED. g_idx values outside [0, K/groupsize) give
 * Q4_ERR_INVALID_ARG.
 *
 * Ownership: the inputs are read (the call synchronizes the device) and
 * copied into handle-owned device memory in private layouts: the packed
 * weights at the same size (K rounded up to a multiple of 128 rows), and
 * each group's scale and zero point as one 32-bit word per column (the
 * checkpoint's scale and packed zero tensors are not kept). The caller
 * keeps and may free or change its tensors afterwards; such changes do not
 * reach the handle (make a new one). The handle also owns the skinny
 * kernel's split-K workspace, sized for the largest splits x M its launch
 * plan takes at any M <= Q4_GEMV_MAX_M (none when the plan never splits K,
 * as for 4096-wide and wider layers on 256 CUs). It never holds a
 * dequantized K x N matrix. Temporary device buffers for the checkpoint's
 * group parameters are allocated and freed during the call.
 *
 * Returns NULL on error (q4_last_status / q4_last_error tell why).
 */
q4_matrix* q4_make(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                   const int32_t* g_idx, int K, int N, int groupsize);

/*
 * q4_make_bits -- q4_make for 4- or 8-bit codes (bits = 4 or 8). GPTQModel
 * wiki "Inference Backends": GPTQ kernels declare 4- and 8-bit weights
 * (backend catalogue) and the native 8-bit GPTQ path keeps the same
 * checkpoint tensors (section "Runtime cache lifetime"). With bits = 8 a word
 * holds four codes packed the same way (code i in bits 8i .. 8i + 7):
 * qweight [K/4][N] (row k = 4r + i in byte i of word (r, n)), qzeros
 * [K/groupsize][N/4] (column n = 4c + j in byte j of word (g, c)); a NULL
 * qzeros means the symmetric zero point 2^(8-1) = 128. bits = 4 is q4_make.
 * Every other argument, the ownership and the errors are as in q4_make
 * (Q4_ERR_UNSUPPORTED for other bit widths). The matmul calls are the same;
 * 8-bit handles take at most two skinny-kernel column tiles and GEMM
 * variant 0 or 3 only.
 */
q4_matrix* q4_make_bits(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                        const int32_t* g_idx, int K, int N, int groupsize, int bits);

/*
 * q4_matmul -- out[M][N] = fp16(x[M][K] @ W) (Lorax page, Description: x @ q4
 * producing (batch, width)). Accumulation is in fp32 (GPTQModel wiki,
 * hardware table, ExLlama v2 row: FP32 accumulation, FP16 scales); the only
 * rounding to fp16 is the final cast (round to nearest even).
 *
 * x and out are caller-owned device buffers and must not overlap. M == 0 is
 * a no-op returning Q4_OK. M < 0, NULL pointers or a NULL handle give
 * Q4_ERR_INVALID_ARG. M <= Q4_GEMV_MAX_M runs the skinny kernel, larger M the
 * MFMA GEMM (q4_path_for tells which). Sizes beyond the kernels' 32-bit
 * offsets give Q4_ERR_UNSUPPORTED: M * K * 2 or M * N above 2^31 - 1, or
 * more than 2^30 GEMM (output tile, 64-row k-step) pairs (about
 * M * K * N / 2^19).
 *
 * Concurrency: the handle's workspace is shared by its calls, so calls on one
 * handle must be ordered on one stream (or synchronized); different handles
 * are independent. The GEMM's stream-K partial sums (tiles whose K range is
 * split between two workgroups) go to a workspace per (device, stream) that
 * the library allocates on the first call on that stream that needs it
 * (2 x 128 KiB + 4 bytes per workgroup: 128 MiB for 512 workgroups) and
 * keeps until the process ends; calls on one stream share it in order. A
 * captured call keeps the workspace of the stream it was captured on, while
 * a graph replays on whatever stream launches it: graphs holding GEMM calls
 * captured on one stream (torch captures every graph on one shared side
 * stream unless told otherwise) must not be replayed concurrently with each
 * other or with uncaptured GEMM calls on that stream, or they race on its
 * partial sums and arrival counters (wrong outputs, no error). Replays in
 * stream order, one after the other, are safe.
 *
 * Act-order (non-trivial g_idx): the weights are stored in sorted-group
 * order, so the product needs the activations x[:, perm] (the Lorax GPTQ
 * Exllama V1 page, Description: a temporary buffer reorders the activations
 * in the act-order case). Without K splits and for M <= 2, the skinny kernel
 * builds them in LDS itself when they fit (q4_gemv_gather); otherwise, and
 * for the GEMM, a separate kernel first writes x[:, perm] to the handle's
 * workspace.
 *
 * Graph capture: a call may be captured into a HIP graph and replayed; it
 * enqueues kernels only (no memset or copy nodes; the skinny kernel's split-K
 * counters, and the GEMM's stream-K counters, are reset by the kernels). A
 * GEMM call captured on a stream that has no stream-K workspace yet runs one
 * workgroup per output tile instead (the same result up to fp32 rounding).
 * An act-order handle grows its activation workspace on the first call with
 * a larger M that needs the separate permute, which cannot happen under
 * capture: such a call returns Q4_ERR_INVALID_ARG, so make one uncaptured
 * call with the largest M first. Outgrown workspaces are not freed before
 * the handle (act-order buffer) or the process (stream-K buffers), so graphs
 * captured earlier stay valid.
 */
q4_status q4_matmul(const q4_matrix* h, const uint16_t* x, uint16_t* out, int M,
                    hipStream_t stream);

/*
 * q4_matmul_bias -- as q4_matmul, plus bias[n] added to the fp32 accumulator
 * before the single cast to fp16 (GPTQModel wiki, section "Numeric epilogues
 * and input gradients": the bias is summed in FP32 with the product, and the
 * result is rounded once at the end). bias may be NULL (then identical to
 * q4_matmul).
 */
q4_status q4_matmul_bias(const q4_matrix* h, const uint16_t* x, const uint16_t* bias,
                         uint16_t* out, int M, hipStream_t stream);

/*
 * q4_matmul_ex -- q4_matmul_bias with explicit kernel choice, for tests and
 * tuning. path = 0 (automatic, as q4_matmul), Q4_PATH_GEMV (needs
 * 1 <= M <= Q4_GEMV_MAX_M) or Q4_PATH_MFMA (any M >= 1).
 *   skinny kernel: variant = 16-column MFMA tiles per wave, 0 (planned), 1, 2
 *                  or 4; splits = K splits across workgroups, 0 (planned) or
 *                  1..16;
 *   GEMM:          variant = the tile width: 0 or 3 (planned,
 *                  q4_plan_gemm_waves), 4 (128 columns, four waves) or 8
 *                  (256 columns, eight waves; M > 512 only); splits =
 *                  workgroups: 0 (planned, q4_plan_gemm for the planned
 *                  width; for an explicit width, the plan at that width),
 *                  1 (one per output tile: 256 or 64 rows by the width) or
 *                  2..Q4_GEMM_MAX_WORKERS (the tiles' 64-row k-steps shared
 *                  evenly, stream-K; a count above the number of (tile,
 *                  k-step) pairs is reduced to it; under stream capture only
 *                  once the stream has a workspace that large, else
 *                  Q4_ERR_INVALID_ARG).
 * Anything else is Q4_ERR_INVALID_ARG. Results differ between paths,
 * tile widths and split counts only by fp32 rounding. An explicit skinny-kernel
 * split count above the largest the plan takes for the handle grows its
 * split-K workspace, which cannot happen under stream capture
 * (Q4_ERR_INVALID_ARG there: make one uncaptured call with that count first).
 */
q4_status q4_matmul_ex(const q4_matrix* h, const uint16_t* x, const uint16_t* bias,
                       uint16_t* out, int M, int path, int variant, int splits,
                       hipStream_t stream);

/* Bytes of the per-GPU scratch array q4_matmul_static works in (64 MiB). */
#define Q4_STATIC_SCRATCH_BYTES (64u << 20)

/*
 * q4_matmul_static -- q4_matmul_bias for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. It allocates nothing (no hipMalloc, hipFree or allocating
 * library call): every workspace the call needs (the skinny kernel's split-K
 * partial sums and arrival counters, an act-order layer's permuted
 * activations, the GEMM's stream-K partial sums and counters) lives in one
 * static array of Q4_STATIC_SCRATCH_BYTES per GPU. The array is set up when
 * the first handle is made on a GPU (q4_make looks up its device address, at
 * which point the HIP runtime places it in device memory, and clears its
 * counters) and is kept until the process ends.
 *
 * Arguments, result, numerics and errors as q4_matmul_bias (fp16 x, bias,
 * out). The launch plan is q4_matmul_bias's, except that the skinny kernel's
 * K splits are halved, and the GEMM's stream-K workgroups reduced, until
 * their partial sums fit the array (results then differ from q4_matmul_bias
 * only by fp32 rounding; with the plans of the 7B and 70B layers they are the
 * same bits). An act-order call that needs the separate permute (M > 2, or K
 * split) stores x[:, perm] in the array too: M * K * 2 bytes must fit in
 * Q4_STATIC_SCRATCH_BYTES - 64 KiB, else Q4_ERR_UNSUPPORTED with nothing
 * enqueued.
 *
 * Concurrency: every q4_matmul_static call on a GPU shares that GPU's array,
 * which keeps the last call's contents, so calls that overlap in time on one
 * GPU (other streams, concurrent graph replays) race and give wrong results
 * without an error; order them on one stream. Every call leaves the arrival
 * counters at zero.
 */
q4_status q4_matmul_static(const q4_matrix* h, const uint16_t* x, const uint16_t* bias,
                           uint16_t* out, int M, hipStream_t stream);

/*
 * q4_matmul_bf16 -- q4_matmul_bias with bfloat16 activations, bias and output
 * (GPTQModel wiki "Inference Backends", hardware table, ExLlama v2 row: the
 * activation dtype -- FP16, BF16 or FP32 -- is kept, with FP16 scales and
 * FP32 accumulation). x is bfloat16 [M][K], bias bfloat16 [N] or NULL, out
 * bfloat16 [M][N]; the handle (fp16 scales) is the same as for fp16 calls.
 * Accumulation is fp32 and the only rounding of the result is the final
 * round-to-nearest-even cast to bfloat16. The skinny kernel applies the
 * exact weights s * (q - z) (as the fp16 path); the GEMM multiplies the
 * weights rounded once to bfloat16, RNE_bf16(s * (q - z)), since its matrix
 * operands are bfloat16. Same arguments, ownership, errors, concurrency and
 * graph-capture rules as q4_matmul.
 */
q4_status q4_matmul_bf16(const q4_matrix* h, const uint16_t* x, const uint16_t* bias,
                         uint16_t* out, int M, hipStream_t stream);

/*
 * q4_matmul_ex_bf16 -- q4_matmul_bf16 with an explicit kernel, as
 * q4_matmul_ex; the GEMM takes variant 0 or 3 only (other variants:
 * Q4_ERR_UNSUPPORTED).
 */
q4_status q4_matmul_ex_bf16(const q4_matrix* h, const uint16_t* x, const uint16_t* bias,
                            uint16_t* out, int M, int path, int variant, int splits,
                            hipStream_t stream);

/* q4_free -- release a handle and every device buffer it owns (NULL is
 * allowed). The caller must have synchronized every stream that used it. The
 * pages have no counterpart: their handle lives as long as the module holding
 * it; a C ABI needs an explicit end of life. */
void q4_free(q4_matrix* h);

/*
 * q4_last_status / q4_last_error -- the status and the reason of the last
 * failing call on this thread (Q4_OK and "" before any failure). Every
 * failure is returned, never replaced by a slower route: an explicitly
 * requested backend whose checks fail raises rather than silently running
 * another one, and the rejection keeps its specific reason (GPTQModel wiki
 * "Inference Backends", section "Loading and selecting a backend", and the
 * device-validation paragraph of "Hardware, dependency, and format
 * requirements"). The message is thread-local and stays valid until the next
 * failing call on the same thread.
 */
q4_status q4_last_status(void);
const char* q4_last_error(void);
/*
 * q4_make_cat -- one handle over the column concatenation of `parts` layers
 * (1 <= parts <= 64) that take the same input: QKV or gate/up projection
 * fusion (GPTQModel wiki "Inference Backends", section "How AUTO selection
 * works": eligible QKV or gate/up calls are combined into one after backend
 * selection). One q4_matmul then computes all parts with one launch.
 *
 * Arguments: arrays of `parts` device pointers qweight[i] [K/8][N[i]],
 * qzeros[i] [K/groupsize][N[i]/8], scales[i] [K/groupsize][N[i]] (layouts as
 * in q4_make; qzeros[i] NULL, or qzeros itself NULL, for symmetric parts);
 * N[i] > 0 and a multiple of 8 (host array); one g_idx shared by every part
 * (NULL allowed), K and groupsize as in q4_make.
 *
 * The handle behaves as one layer with N = sum N[i] columns: output column
 * off_i + n (off_i = N[0] + ... + N[i-1]) is column n of part i, and a bias
 * passed to q4_matmul_bias is the concatenation of the parts' biases. Each
 * column's result is the one a handle of its own part gives (same kernel,
 * same order of accumulation when the plan takes the same K splits).
 * Ownership and errors as q4_make; every part's arguments are checked.
 */
q4_matrix* q4_make_cat(int parts, const int32_t* const* qweight, const int32_t* const* qzeros,
                       const uint16_t* const* scales, const int32_t* g_idx, int K, const int* N,
                       int groupsize);

/* q4_make_cat_bits -- q4_make_cat for 4- or 8-bit parts (all parts the
 * same width; layouts as in q4_make_bits). */
q4_matrix* q4_make_cat_bits(int parts, const int32_t* const* qweight, const int32_t* const* qzeros,
                            const uint16_t* const* scales, const int32_t* g_idx, int K, const int* N,
                            int groupsize, int bits);

/*
 * q4_path_for -- the kernel q4_matmul would launch for this M (Q4_PATH_*),
 * or -1 for a NULL handle or M < 0. Lets a caller check which kernel runs
 * ("GPTQ's 'Exllama Kernel Not Installed' Warning": check which kernel runs
 * rather than relying on the absence of a warning).
 */
int q4_path_for(const q4_matrix* h, int M);

/*
 * q4_dequant_dump -- debug: run the unpack + dequantize code of kernel `path`
 * (the dequantized values a kernel computes, dumped in a debug mode so that
 * the in-register unpack and dequantization of "GPTQ's 'Exllama Kernel Not
 * Installed' Warning", section "What the fallback actually does", can be
 * compared bit for bit with the plain definition s * (q - z)):
 * kernel Q4_PATH_GEMV or Q4_PATH_MFMA, over the whole handle, writes the fp16
 * values that kernel feeds its multiply-accumulate to w[K][N] (device
 * buffer, caller-owned, original k order). Each value is
 * round-to-nearest-even of s * (q - z). Not on the hot path.
 */
q4_status q4_dequant_dump(const q4_matrix* h, int path, uint16_t* w, hipStream_t stream);

/*
 * q4_dequant_dump_bf16 -- as q4_dequant_dump (same purpose and source) for
 * the bfloat16 kernels: w is
 * bfloat16 [K][N]. Q4_PATH_GEMV: the skinny kernel's q - z in bfloat16 times
 * the fp32 scale, rounded once to bfloat16; Q4_PATH_MFMA: the bfloat16
 * weights the GEMM feeds its MFMA. Each value is round-to-nearest-even of
 * s * (q - z) to bfloat16.
 */
q4_status q4_dequant_dump_bf16(const q4_matrix* h, int path, uint16_t* w, hipStream_t stream);

/*
 * q4_gemv_gather -- 1 when, for this act-order handle, M and K splits
 * (0: the automatic plan), the skinny kernel builds x[:, perm] in LDS itself,
 * 0 when q4_matmul runs the separate permute kernel first (and for handles
 * without act-order). -1 for a NULL handle, M outside [1, Q4_GEMV_MAX_M] or
 * splits outside [0, 16].
 */
int q4_gemv_gather(const q4_matrix* h, int M, int splits);

/* Handle geometry: K, N, groupsize (after -1 -> K), act-order flag (1 when a
 * non-trivial g_idx was given). Returns 0, or -1 for a NULL handle. */
int q4_handle_info(const q4_matrix* h, int* K, int* N, int* groupsize, int* act_order);

/* The handle's code width (4 or 8), or -1 for a NULL handle. */
int q4_handle_bits(const q4_matrix* h);

/*
 * q4_read_probe -- measurement helper, not part of the product: enqueue one
 * kernel on `stream` that reads `bytes` of device memory at buf with the
 * skinny kernel's kind of load (16 bytes a lane, non-temporal) and no other
 * work, so that timing it gives the achievable read rate of one launch of
 * that size. Decode steps whose bytes are mostly weights run at the speed of
 * memory, not arithmetic ("GPTQ's 'Exllama Kernel Not Installed' Warning",
 * section "What the fallback actually does"); this is the ceiling the fused
 * kernel's effective bandwidth is compared with. buf: device pointer, 16-byte aligned; bytes: a positive
 * multiple of 16384; sink: device buffer of 256 uint32_t, written only when
 * the folded data match a fixed constant (the caller ignores it). Returns
 * Q4_ERR_INVALID_ARG for bad arguments (nothing enqueued), Q4_ERR_HIP if the
 * launch fails.
 */
q4_status q4_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Host-only planning helpers (no HIP calls; usable without a GPU).
 * ---------------------------------------------------------------------- */

/*
 * q4_check_shape -- the argument checks q4_make applies to (K, N, groupsize),
 * without touching memory. Returns Q4_OK, Q4_ERR_INVALID_ARG or
 * Q4_ERR_UNSUPPORTED (message in q4_last_error).
 */
q4_status q4_check_shape(int K, int N, int groupsize);

/* q4_check_shape for q4_make_bits (bits = 4 or 8; other widths give
 * Q4_ERR_UNSUPPORTED). */
q4_status q4_check_shape_bits(int K, int N, int groupsize, int bits);

/*
 * q4_plan_actorder -- host act-order plan for a host copy of g_idx[K]:
 * perm[k'] = stable argsort of g_idx (ties by increasing k), *trivial = 1
 * when g_idx[k] == k / groupsize for all k (perm is then the identity).
 * Returns Q4_ERR_INVALID_ARG for out-of-range values and Q4_ERR_UNSUPPORTED
 * when the sorted groups are not exactly groupsize rows each.
 */
q4_status q4_plan_actorder(const int32_t* g_idx_host, int K, int groupsize, int32_t* perm,
                           int* trivial);

/*
 * q4_plan_gemm -- the streaming GEMM's planned workgroup count for an
 * M x N output with K rows on a chip of num_cu compute units (<= 0: 256), at
 * the planned tile width for 4-bit weights (q4_plan_gemm_waves; an 8-bit
 * handle plans as for four waves). Output tiles are 64 x 128
 * when M <= 512, else 256 x 128 (four waves) or 256 x 256 (eight waves).
 * Four waves: one workgroup per tile when the tiles fill whole rounds of two
 * per CU (to within a tenth) or make at least 1.5 such rounds; otherwise the
 * tiles' 64-row k-steps are shared evenly (stream-K): with 64-row tiles by
 * 2 num_cu workgroups when each gets at least 32 k-steps, by num_cu when
 * each gets at least 16, else by one per 16 k-steps (at least one per tile);
 * with 256-row tiles by min(2 num_cu, max(2 tiles, num_cu)). Eight waves
 * (one workgroup per CU): one per tile when the tiles fill whole rounds of
 * num_cu to within a tenth, else num_cu. Never more than there are (tile,
 * k-step) pairs.
 * Host-only; -1 for M, N or K < 1.
 */
int q4_plan_gemm(int M, int N, int K, int num_cu);

/*
 * q4_plan_gemm_waves -- the streaming GEMM's planned tile width, in waves of
 * 32 columns: 8 (256-column tiles) for M > 512 when the 256 x 256 tiles are
 * at least num_cu, or at least num_cu / 2 with at least 64 (tile, 64-row
 * k-step) pairs per CU, or any number with at least 128 pairs per CU; else
 * 4 (128-column tiles). For 4-bit weights: 8-bit handles always take 4.
 * Host-only; -1 for M, N or K < 1.
 */
int q4_plan_gemm_waves(int M, int N, int K, int num_cu);

/*
 * q4_plan_gemv -- the skinny kernel's launch plan for (M, K, N, groupsize) on
 * a chip of num_cu compute units (<= 0: 256): 16-column tiles per wave
 * (*col_tiles: 1, 2 or 4) and K splits across workgroups (*splits: 1..16).
 * Host-only. Q4_ERR_INVALID_ARG for M outside [1, Q4_GEMV_MAX_M] or null
 * outputs; the q4_check_shape status for an unsupported shape.
 */
q4_status q4_plan_gemv(int M, int K, int N, int groupsize, int num_cu, int* col_tiles,
                       int* splits);

/*
 * q4_plan_gemv_gather -- host-only form of q4_gemv_gather's rule: 1 when
 * splits == 1, M <= 2, K padded to whole 128-row blocks is at most 12288
 * rows and M of those rows, each padded by 8 halfs, fit 20480 halfs (40 KiB
 * of LDS); else 0. -1 for M outside [1, Q4_GEMV_MAX_M], K < 1 or splits outside
 * [1, 16].
 */
int q4_plan_gemv_gather(int M, int K, int splits);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
