// Skinny fused GPTQ kernel for 1 <= M <= 32 (decode and small batches).
//
// q4_gemv_kernel<NGB, CT, XS, TAIL, XL, BF, W8, MB, R1>: NGB groups per
// 128-row block, CT 16-column tiles per wave, XS k-steps per activation load,
// TAIL (K not a multiple of 128), XL (act-order activations staged in LDS),
// BF (bfloat16 activations and output), W8 (8-bit codes; 4-bit otherwise),
// MB blocks of 16 activation rows (1 for M <= 16; 2 for 16 < M <= 32, which
// load one k-step per activation load and share each unpacked weight
// fragment between the two row blocks' MFMAs), R1 (M = 1: one-row mode,
// below). (Four row blocks, M <= 64,
// measured 1.4-2.5x slower than the GEMM on the 7B and 70B MLP shapes: their
// activation registers leave room for two column tiles at one workgroup per
// CU, and the activation loads grow with every row block.)
//
// When the weights dominate the bytes moved, the speed of a decode step is
// set by HBM bandwidth, not by arithmetic ("GPTQ's 'Exllama Kernel Not
// Installed' Warning", section "What the fallback actually does"). So the
// kernel reads each packed word once with 16-byte loads, turns it into
// fp16 values in registers and never stores a dequantized weight.
//
// Mapping. A workgroup of 8 waves owns CT 16-column tiles (16 * CT output
// columns); its waves split its K range in whole 128-row k-blocks.
//  * lane l works on column c = l % 16 of every tile and on k-block quarter
//    kb = l / 16. One 16-byte load of the private layout (chunk (b, kb, c))
//    gives it the eight rows 32 * (4b + i) + 8 * kb .. +7 for each of the
//    four k-steps i of block b, which is exactly the B operand of four
//    v_mfma_f32_16x16x32_f16 (lane l: rows 8 * (l / 16) .. +7 of column
//    l % 16). (8-bit codes: the chunk is 32 bytes, two 16-byte loads.)
//    A is the activations (row m = l % 16), shared by the CT tiles.
//    M is padded to 16 on the matrix pipe, which has the capacity to spare:
//    output rows m >= M are never stored, so what A holds in those rows does
//    not matter. That lets one 16-byte load serve XS = 16 / R k-steps when
//    M <= R (R = 4 or 8): lane group s of each 16-lane row loads the R rows of
//    k-step s, and a DPP row shift moves them into lanes 0 .. R-1 for that
//    step's MFMA, instead of one mostly empty load per k-step.
//  * One-row mode (M = 1, R1): no shift at all. Every k-step's MFMA takes the
//    activation register as loaded, so A row 4s holds k-step s's activations
//    and output row 4s of k-step i's product is x . W_i only for s = i. Each
//    k-step's product starts from zero and only that row (the first element
//    of lane group i) is folded into its own total; the four lane groups'
//    totals are added in the cross-wave sum. That saves the twelve row shifts
//    of a block (58 -> 42 vector instructions with the packed zero points
//    below) and leaves the four products independent of each other.
//  * B is the exact small integers q - z in fp16, and the per-group scale is
//    applied once per group to the fp32 MFMA sum:
//    sum_k x * s * (q - z) = s * sum_k x * (q - z). The weight s * (q - z) is
//    exact in fp32, so this is the product with the exact dequantized weight,
//    accumulated in fp32, and the vector ALU does one unpack and one packed
//    subtract per two weights. (BF: the same exact q - z as bfloat16, formed
//    by one fused multiply-add per value; the MFMA takes bfloat16.)
//  * the weights are read exactly once, with the non-temporal hint (5-7%
//    faster on the 7B layers than default caching), and so are the group
//    words (5-6% faster on the 7B layers than cached loads of them, 1%
//    slower on the 70B MLP layers);
//  * each wave keeps D k-blocks of loads in flight (a ring of register
//    buffers, refilled as soon as a block is multiplied), so a CU has
//    8 waves x D x 1 KiB x CT of weights outstanding. Every load takes a
//    fixed per-lane offset plus a wave-uniform offset in a scalar register,
//    so the loop spends its vector instructions on the unpack alone;
//  * the waves' fp32 results are summed in LDS in wave order;
//  * grid.y splits K across workgroups when the column tiles alone cannot
//    give every CU a workgroup. Each split writes fp32 partials; the last
//    workgroup of a column tile to arrive (counted with an agent-scope
//    atomic) sums them in split order, so the result does not depend on
//    timing. Reductions stay in fp32 (GPTQModel wiki "Inference Backends",
//    section "Numeric epilogues": FP32 split/tile reductions, bias added
//    before the single cast).
//
// Act-order. The weights are stored in sorted-group order, so k-step rows
// need the activations x[:, perm] (the Lorax GPTQ Exllama V1 page,
// Description: a temporary buffer reorders the activations in the act-order
// case). When K is not split, M <= 2 and x fits, each workgroup builds that
// permuted copy in LDS itself instead of a separate permute launch (XL):
// every thread loads 16-byte chunks of x in the original order (eight rows
// k of one activation row) and the sorted positions inv[k] of those rows,
// issues the ring's first weight loads, and then writes each half to its
// sorted position in LDS. The loads are contiguous and independent, so they
// travel with the weights; only the LDS stores scatter. (Gathering
// x[m][perm[k']] from memory instead costs a scattered 2-byte load per
// element in every workgroup.) The loop then reads its A operands from LDS.
// Rows from K to the end of the last block are stored as zeros.
#include "q4_device.h"
#include "q4_internal.h"

namespace {

using namespace q4dev;

constexpr int WV = q4::kGemvWaves;     // waves per workgroup
constexpr int NT = 64 * WV;            // threads per workgroup
// k-blocks in flight per wave: kGemvDepth for one column tile and one row
// block, half that for wider tiles or more row blocks (their buffers are
// larger; this keeps two workgroups per CU for M <= 16 and the register file
// unspilled for M > 16).
template <int CT, int MB>
constexpr int depth() { return (CT >= 2 || MB > 1) ? q4::kGemvDepth / 2 : q4::kGemvDepth; }

struct GemvArgs {
    const uint32_t* qweight;
    const uint32_t* sz;     // [ng][N]: scale bits | zero << 16
    const uint16_t* x;
    const uint16_t* inv;    // act-order: original row -> sorted position (XL)
    const uint16_t* bias;
    uint16_t* out;
    float* partials;
    uint32_t* counters;
    int M, K, N, G;
    int ng;                 // K / G
    int gshift;             // group of k-step t (32 rows) = t >> gshift (31: one group)
    int kblocks;            // ceil(K / 128)
    int blocks_per_split;
    int blocks_per_wave;
    int splits;
    int ldx;                // XL: halfs per LDS activation row (kblocks * 128 + pad)
};

// One k-block of loads for one lane. NGB = groups per block: 4 (groups of 32
// rows), 2 (64) or 1 (128, 256, or one group over K). W8: 8-bit codes, whose
// block takes two 16-byte loads per column (WL = 2).
template <bool W8>
constexpr int wl() { return W8 ? 2 : 1; }

template <int NGB, int CT, bool W8, int MB>
struct Block {
    u4 w[CT][wl<W8>()];
    u4 a[MB][4];            // row block r: activation rows 16 r + (lane % 16)
    uint32_t sz[NGB][CT];   // scale bits | zero << 16
};

// Per-lane byte offsets, fixed for the whole kernel; each block adds a
// wave-uniform offset held in a scalar register. Columns past N read column
// N - 1 (their results are never stored); activation rows m >= M lie past the
// end of x and read zeros.
template <int CT>
struct Lane {
    uint32_t w[CT];          // chunk (kb, n_j) of a block * 16 (8-bit: * 32)
    uint32_t sz[CT];         // n_j * 4
    uint32_t x;              // ((l % R) * K + 8 * kb + 32 * ((l % 16) / R)) * 2
};

// Descriptors of the tensors, and one of size 0: a load through it
// returns zeros and moves no data. Only the last k-block of a K that is not a
// multiple of 128 needs it (TAIL): its k-steps past K and its groups past K / G.
struct Rsrc {
    rsrc_t w, x, sz, none, inv;
};

// Load k-block b (0 <= b < kblocks). The per-block offsets are wave-uniform
// (scalar registers; the k-step offset 64 i of the activations folds into the
// instruction's immediate offset).
// XS = k-steps per activation load (1, 2 or 4); B.a[0 .. 4/XS - 1] are loaded.
// XL: the activations come from the workgroup's LDS copy instead; they are
// read when the block is multiplied.
template <int NGB, int CT, int XS, bool TAIL, bool XL, bool W8, int MB>
__device__ __forceinline__ void load_block(Block<NGB, CT, W8, MB>& B, const GemvArgs& p, const Rsrc& r,
                                           const Lane<CT>& ln, int b)
{
    const uint32_t wso = (uint32_t)b * (uint32_t)p.N * 64u * wl<W8>();
#pragma unroll
    for (int j = 0; j < CT; ++j)
#pragma unroll
        for (int v = 0; v < wl<W8>(); ++v) B.w[j][v] = buf_load16_nt(r.w, ln.w[j] + 16u * v, wso);
    const int ksteps = p.K >> 5;
    if constexpr (!XL) {
        // (row block rb starts 16 rb rows, 32 rb K bytes, further into x;
        // rows past M lie past its end and read zeros)
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
#pragma unroll
            for (int i = 0; i < 4 / XS; ++i) {
                const rsrc_t rx = (!TAIL || 4 * b + i < ksteps) ? r.x : r.none;
                B.a[rb][i] = buf_load16(rx, ln.x + (uint32_t)rb * 32u * (uint32_t)p.K + 64u * XS * i,
                                        (uint32_t)b * 256u);
            }
    }
#pragma unroll
    for (int gi = 0; gi < NGB; ++gi) {
        const int g = (4 * b + gi * (4 / NGB)) >> p.gshift;
        const bool ok = !TAIL || g < p.ng;
        const rsrc_t rsz = ok ? r.sz : r.none;
#pragma unroll
        for (int j = 0; j < CT; ++j) B.sz[gi][j] = buf_load4_nt(rsz, ln.sz[j], (uint32_t)g * (uint32_t)p.N * 4u);
    }
}

// Rows shifted down a 16-lane row by SH lanes (DPP row_shl; lanes past the
// end of the row read zero).
template <int SH>
__device__ __forceinline__ u4 row_shl(u4 v)
{
    u4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (uint32_t)__builtin_amdgcn_mov_dpp((int)v[e], 0x100 + SH, 0xF, 0xF, true);
    return o;
}

// The A operand of k-step i: with XS > 1, rows 0 .. R-1 (R = 16 / XS) come
// from lane group i % XS of the load that holds step i, shifted down the row.
// (i is a constant after unrolling, so the switch folds away.)
template <int XS>
__device__ __forceinline__ u4 a_operand(const u4 a[4], int i)
{
    constexpr int R = 16 / XS;
    const u4 v = a[i / XS];
    switch (R * (i % XS)) {
    case 4: return row_shl<4>(v);
    case 8: return row_shl<8>(v);
    case 12: return row_shl<12>(v);
    default: return v;
    }
}

// Multiply one block into the totals: per group, the MFMA sums of x * (q - z)
// over its k-steps, then tot += s * sum in fp32. BF: bfloat16 activations and
// the exact q - z as bfloat16 (both operands bfloat16 on the matrix pipe).
// XL: block b's activations are read from the LDS copy (xl = this lane's
// address in it for the first block of the workgroup's range, bs0).
template <int NGB, int CT, int XS, bool XL, bool BF, bool W8, int MB, bool R1>
__device__ __forceinline__ void compute_block(const Block<NGB, CT, W8, MB>& B, f4 (&tot)[MB][CT],
                                              const char* xl, int b, int bs0, uint32_t magic)
{
    constexpr int SPG = 4 / NGB;   // k-steps per group inside the block
    u4 av[MB][4];
    if constexpr (XL) {
        const char* src = xl + (b - bs0) * 256;
#pragma unroll
        for (int i = 0; i < 4 / XS; ++i) av[0][i] = *reinterpret_cast<const u4*>(src + 64 * XS * i);
    } else {
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
#pragma unroll
            for (int i = 0; i < 4 / XS; ++i) av[rb][i] = B.a[rb][i];
    }
#pragma unroll
    for (int gi = 0; gi < NGB; ++gi) {
        zero_t zp[CT];
        mix_t mz[CT];
        float sf[CT];
        // (1 kept opaque, so that f * h + c stays one v_fma_mix_f32 instead
        // of a conversion and an add)
        float one = 1.0f;
        if constexpr (BF) asm("" : "+v"(one));
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            if constexpr (BF) mz[j] = mix_consts(B.sz[gi][j] >> 16, one, magic);
            else zp[j] = zero_pair_sz(B.sz[gi][j], magic);
            sf[j] = f16_bits_to_f32((uint16_t)B.sz[gi][j]);
        }
        f4 acc[MB][CT];
        f4 pr[R1 ? SPG : 1][CT];   // one-row mode: the group's k-step products
#pragma unroll
        for (int ii = 0; ii < SPG; ++ii) {
            const int i = gi * SPG + ii;
            const f4 c0 = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < CT; ++j) {
                // the B operand of tile j at k-step i, unpacked once for the
                // MB row blocks
                u4 bw;
                if constexpr (W8) {
                    // k-step i: words 2i, 2i + 1 of the lane's 32-byte chunk
                    const uint32_t w0 = B.w[j][i >> 1][2 * (i & 1)], w1 = B.w[j][i >> 1][2 * (i & 1) + 1];
                    if constexpr (BF) bw = bitcast<u4>(mix_word8(w0, w1, mz[j]));
                    else bw = bitcast<u4>(sub_zero_word8(w0, w1, zp[j]));
                } else if constexpr (BF) {
                    bw = bitcast<u4>(mix_word(B.w[j][0][i], mz[j]));
                } else {
                    bw = bitcast<u4>(sub_zero_word(B.w[j][0][i], zp[j]));
                }
                if constexpr (R1) {
                    // One row: the activation register as loaded (lane group
                    // s holds k-step s) against k-step i's weights. Output
                    // row 4s of this product is x . W_i only for s = i: lane
                    // group i's first element. Each k-step gets its own
                    // product from zero and its own total, tot[0][j][i]; the
                    // other rows are never read.
                    if constexpr (BF) pr[ii][j] = mfma16(bitcast<b8>(av[0][0]), bitcast<b8>(bw), c0);
                    else pr[ii][j] = mfma16(bitcast<h8>(av[0][0]), bitcast<h8>(bw), c0);
                } else {
#pragma unroll
                    for (int rb = 0; rb < MB; ++rb) {
                        const u4 a = a_operand<XS>(av[rb], i);
                        if constexpr (BF) acc[rb][j] = mfma16(bitcast<b8>(a), bitcast<b8>(bw), ii == 0 ? c0 : acc[rb][j]);
                        else acc[rb][j] = mfma16(bitcast<h8>(a), bitcast<h8>(bw), ii == 0 ? c0 : acc[rb][j]);
                    }
                }
            }
        }
        if constexpr (R1) {
            // (after all of the group's products, so that the matrix pipe
            // runs them back to back)
#pragma unroll
            for (int ii = 0; ii < SPG; ++ii)
#pragma unroll
                for (int j = 0; j < CT; ++j)
                    tot[0][j][gi * SPG + ii] = __builtin_fmaf(sf[j], pr[ii][j][0], tot[0][j][gi * SPG + ii]);
            // (the products' other registers stay allocated until here, past
            // the read above, which waits for the matrix pipe; reused
            // earlier, each reuse would wait for the product's last write)
#pragma unroll
            for (int ii = 0; ii < SPG; ++ii)
#pragma unroll
                for (int j = 0; j < CT; ++j) asm volatile("" ::"v"(pr[ii][j]));
        } else {
#pragma unroll
            for (int rb = 0; rb < MB; ++rb)
#pragma unroll
                for (int j = 0; j < CT; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) tot[rb][j][e] = __builtin_fmaf(sf[j], acc[rb][j][e], tot[rb][j][e]);
        }
    }
}

// Act-order staging (XL). Thread tid owns the 8-row units u = tid + NT * j
// (j < XJ) of the original order: iv[j] holds inv[8u .. 8u + 7], xv[j][i]
// the activations x[m0 + i][8u .. 8u + 7]. Rows m >= M lie past the end of x
// (the loads return zeros) and units past K are not stored.
constexpr int XR = 2;   // activation rows per staging round

template <int XJ>
__device__ __forceinline__ void stage_load(u4 (&xv)[XJ][XR], const GemvArgs& p, const Rsrc& r, int tid, int m0)
{
#pragma unroll
    for (int i = 0; i < XR; ++i)
#pragma unroll
        for (int j = 0; j < XJ; ++j)
            xv[j][i] = buf_load16(r.x, ((uint32_t)(m0 + i) * (uint32_t)p.K + 8u * (uint32_t)(tid + NT * j)) * 2u);
}

template <int XJ>
__device__ __forceinline__ void stage_store(uint16_t* xs, const u4 (&xv)[XJ][XR], const u4 (&iv)[XJ],
                                            const GemvArgs& p, int tid, int m0)
{
    const int units = p.K >> 3;
#pragma unroll
    for (int i = 0; i < XR; ++i)
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            if (m0 + i >= p.M || tid + NT * j >= units) continue;
            uint16_t* row = xs + (size_t)(m0 + i) * p.ldx;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                row[(iv[j][e >> 1] >> (16 * (e & 1))) & 0xFFFFu] = (uint16_t)(xv[j][i][e >> 1] >> (16 * (e & 1)));
        }
}

// The kernel takes the fields its first loads need as separate leading
// arguments (the same values as in `args`): the build asks the compiler to
// preload leading scalar kernel arguments into SGPRs, which the hardware
// fills before the waves start, so the first weight loads need not wait for
// a fetch of the argument segment (a struct argument is never preloaded).
// Measured on the read probe: 0.05-0.1 us less per launch.
template <int NGB, int CT, int XS, bool TAIL, bool XL, bool BF, bool W8, int MB, bool R1>
__global__ __launch_bounds__(NT) void q4_gemv_kernel(const uint32_t* qweight, const uint32_t* sz,
                                                      const uint16_t* x, int M, int K, int N, int kblocks,
                                                      int blocks_per_split, int blocks_per_wave, int gshift,
                                                      int ng, GemvArgs args)
{
    static_assert(!R1 || (XS == 4 && MB == 1), "one-row mode reads four k-steps per activation load");
    constexpr int COLS = 16 * CT;
    static_assert(NT % COLS == 0, "a thread's epilogue elements share one column");
    constexpr int ROWS = 16 * MB;
    __shared__ float red[WV][ROWS][COLS];
    __shared__ int last_flag;
    extern __shared__ u4 xs_dyn[];   // XL: the workgroup's activations, [M][ldx] halfs

    GemvArgs p = args;
    p.qweight = qweight;
    p.sz = sz;
    p.x = x;
    p.M = M;
    p.K = K;
    p.N = N;
    p.kblocks = kblocks;
    p.blocks_per_split = blocks_per_split;
    p.blocks_per_wave = blocks_per_wave;
    p.gshift = gshift;
    p.ng = ng;
    const int tid = threadIdx.x;
    // The wave index is uniform across the wave; saying so keeps the block
    // bookkeeping in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int kb = lane >> 4;
    const int c16 = lane & 15;
    // Workgroup i runs on XCD i % 8 (round-robin dispatch). Neighbouring
    // tiles share the cache lines of their scales and packed zeros (a 128-byte
    // line holds 64 columns of scales, 256 of zeros), and the XCDs' L2 caches
    // are separate, so each XCD takes a contiguous run of tiles.
    const int T = (p.N + COLS - 1) / COLS;   // (the grid's x size, without a hidden-argument load)
    const int tile = (T & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (T >> 3) + (int)(blockIdx.x >> 3);
    const int n0 = tile * COLS;

    Rsrc r;
    r.w = make_rsrc(p.qweight, (uint32_t)p.kblocks * (uint32_t)p.N * 64u * wl<W8>());
    r.x = make_rsrc(p.x, (uint32_t)p.M * (uint32_t)p.K * 2u);
    r.sz = make_rsrc(p.sz, (uint32_t)p.ng * (uint32_t)p.N * 4u);
    r.none = make_rsrc(p.qweight, 0u);   // (used by TAIL only)
    if constexpr (XL) r.inv = make_rsrc(p.inv, (uint32_t)p.K * 2u);
    Lane<CT> ln;
#pragma unroll
    for (int j = 0; j < CT; ++j) {
        const int n = min(n0 + 16 * j + c16, p.N - 1);
        ln.w[j] = q4::chunk_in_block(kb, n, p.N) * 16u * wl<W8>();
        ln.sz[j] = (uint32_t)n * 4u;
    }
    constexpr int R = 16 / XS;
    {
        // rows m >= M fall past the end of x and read zeros
        ln.x = ((uint32_t)(c16 % R) * (uint32_t)p.K + 8u * (uint32_t)kb + 32u * (uint32_t)(c16 / R)) * 2u;
    }

    const int split = blockIdx.y;
    const int bs0 = split * p.blocks_per_split;
    const int bs1 = min(bs0 + p.blocks_per_split, p.kblocks);
    const int b0 = bs0 + wave * p.blocks_per_wave;
    const int nb = min(b0 + p.blocks_per_wave, bs1) - b0;   // may be <= 0

    // XL: this lane's A-operand address in the LDS copy for block bs0 = 0
    // (rows m >= M read row M - 1; those output rows are not stored)
    uint16_t* xs = reinterpret_cast<uint16_t*>(xs_dyn);
    const char* xl = reinterpret_cast<const char*>(
        xs + (size_t)min(c16 % R, p.M - 1) * p.ldx + 8 * kb + 32 * (c16 / R));

    f4 tot[MB][CT];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int j = 0; j < CT; ++j) tot[rb][j] = f4{0.f, 0.f, 0.f, 0.f};

    // the unpack's OR constant, kept in a register for the whole loop (as a
    // constant it was rebuilt in every block)
    uint32_t magic = kMagic2;
    asm volatile("" : "+v"(magic));
    constexpr int D = depth<CT, MB>();
    // Ring of D register buffers: block b0 + D * rd + d lives in buf[d].
    // Once a block is multiplied its buffer is refilled with the block D
    // further on. Past the wave's last block the loads repeat that block
    // (addresses stay in range, the data comes from cache) and the last
    // round skips those buffers, so the loop body has no branches and the
    // compiler's wait before each multiply covers exactly that block's
    // loads. sched_barrier keeps each block's loads and arithmetic in
    // program order: the loads issue in the same order in the prologue
    // and in the loop (so the waits at the loop head need not assume the
    // worse of two orders), and no work of a later block (which would
    // wait for its loads) is hoisted into an earlier one.
    const int bl = b0 + nb - 1;
    Block<NGB, CT, W8, MB> buf[D];
    // XL: the first XR activation rows and the sorted positions go out
    // before the weights, so storing them waits for them alone.
    constexpr int XJ = XL ? q4::kGemvXUnits : 1;
    u4 iv[XJ];
    u4 xv[XJ][XR];
    if constexpr (XL) {
#pragma unroll
        for (int j = 0; j < XJ; ++j) iv[j] = buf_load16(r.inv, (uint32_t)(tid + NT * j) * 16u);
        stage_load<XJ>(xv, p, r, tid, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // (With XL the first loads are issued by every wave, so that the staging
    // stores' waits need not cover both a path with and one without them; K
    // is not split then, so block bl = kblocks - 1 exists for a wave without
    // blocks.)
    if (XL || nb > 0) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load_block<NGB, CT, XS, TAIL, XL, W8, MB>(buf[d], p, r, ln, min(b0 + d, bl));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // The bias of the column this thread stores in the epilogues below
    // (column tid % COLS for every element it takes), loaded now so that its
    // latency hides behind the k-loop rather than following the cross-wave
    // sum (after the first weight loads, which need not wait for its
    // pointer). One unconditional load through a descriptor, empty without a
    // bias and ending at column N, so that no branch around it makes the
    // compiler wait for every load in flight at the join.
    const uint16_t bias_h = (uint16_t)buf_load2(make_rsrc(p.bias, p.bias ? (uint32_t)p.N * 2u : 0u),
                                                (uint32_t)(n0 + tid % COLS) * 2u);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (XL) {
        stage_store<XJ>(xs, xv, iv, p, tid, 0);
        for (int m0 = XR; m0 < p.M; m0 += XR) {
            stage_load<XJ>(xv, p, r, tid, m0);
            stage_store<XJ>(xs, xv, iv, p, tid, m0);
        }
        // rows K .. end of the last block
        const int pad = p.kblocks * 128 - p.K;
        for (int idx = tid; idx < p.M * pad; idx += NT) xs[(size_t)(idx / pad) * p.ldx + p.K + idx % pad] = 0;
        __syncthreads();
    }
    if (nb > 0) {
        const int rounds = (nb + D - 1) / D;
        for (int rd = 1; rd < rounds; ++rd) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                compute_block<NGB, CT, XS, XL, BF, W8, MB, R1>(buf[d], tot, xl, b0 + D * (rd - 1) + d, bs0, magic);
                load_block<NGB, CT, XS, TAIL, XL, W8, MB>(buf[d], p, r, ln, min(b0 + D * rd + d, bl));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        const int last = nb - D * (rounds - 1);   // 1 .. D blocks in the last round
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (d < last) compute_block<NGB, CT, XS, XL, BF, W8, MB, R1>(buf[d], tot, xl, b0 + D * (rounds - 1) + d, bs0, magic);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Cross-wave reduction. Lane l holds rows 16 rb + 4 * (l / 16) + i of
    // column l % 16 of each tile (16x16 MFMA output layout). One-row mode:
    // lane group g (= kb) holds row 0's sums over k-steps 4b + g in
    // tot[0][j][g], written to row 4g; the sum below adds the four groups.
    constexpr int LG = R1 ? 4 : 1;   // lane groups holding parts of one row
    if constexpr (R1) {
#pragma unroll
        for (int j = 0; j < CT; ++j) {
            const f4 t = tot[0][j];
            red[wave][4 * kb][16 * j + c16] = kb == 0 ? t[0] : kb == 1 ? t[1] : kb == 2 ? t[2] : t[3];
        }
    } else {
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
#pragma unroll
            for (int j = 0; j < CT; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * rb + 4 * kb + i < p.M) red[wave][16 * rb + 4 * kb + i][16 * j + c16] = tot[rb][j][i];
    }
    __syncthreads();
    // the workgroup's sum for row m, column c (waves in order, then groups)
    auto wg_sum = [&](int m, int c) {
        float y = 0.f;
#pragma unroll
        for (int g = 0; g < LG; ++g) {
            float t = red[0][m + 4 * g][c];
#pragma unroll
            for (int w = 1; w < WV; ++w) t += red[w][m + 4 * g][c];
            y = g == 0 ? t : y + t;
        }
        return y;
    };

    const int n_elems = p.M * COLS;
    if (p.splits == 1) {
        for (int idx = tid; idx < n_elems; idx += NT) {
            const int m = idx / COLS, c = idx % COLS, n = n0 + c;
            if (n >= p.N) continue;
            float y = wg_sum(m, c);
            if (p.bias) y += act_to_f32<BF>(bias_h);
            p.out[(size_t)m * p.N + n] = f32_to_act<BF>(y);
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
    for (int idx = tid; idx < n_elems; idx += NT) {
        const int m = idx / COLS, c = idx % COLS, n = n0 + c;
        if (n >= p.N) continue;
        const float y = wg_sum(m, c);
        __hip_atomic_store(&p.partials[((size_t)split * p.M + m) * p.N + n], y, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        last_flag = (prev == (uint32_t)(p.splits - 1));
    }
    __syncthreads();
    if (!last_flag) return;
    for (int idx = tid; idx < n_elems; idx += NT) {
        const int m = idx / COLS, c = idx % COLS, n = n0 + c;
        if (n >= p.N) continue;
        float y = 0.f;
        for (int s = 0; s < p.splits; ++s)
            y += __hip_atomic_load(&p.partials[((size_t)s * p.M + m) * p.N + n], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        if (p.bias) y += act_to_f32<BF>(bias_h);
        p.out[(size_t)m * p.N + n] = f32_to_act<BF>(y);
    }
    if (tid == 0)
        __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The kernel's leading arguments, then the whole argument struct.
#define Q4_GEMV_ARGS(p)                                                                              \
    (p).qweight, (p).sz, (p).x, (p).M, (p).K, (p).N, (p).kblocks, (p).blocks_per_split, (p).blocks_per_wave, \
        (p).gshift, (p).ng, (p)

template <int NGB, int XS, bool TAIL, bool XL, bool BF, bool W8, int MB, bool R1 = false>
hipError_t launch_ct(const GemvArgs& p, int ct, int splits, hipStream_t stream)
{
    const dim3 block(NT);
    const size_t lds = XL ? (size_t)p.M * p.ldx * 2 : 0;
    switch (ct) {
    case 1: hipLaunchKernelGGL((q4_gemv_kernel<NGB, 1, XS, TAIL, XL, BF, W8, MB, R1>), dim3((p.N + 15) / 16, splits), block, lds, stream, Q4_GEMV_ARGS(p)); break;
    case 2: hipLaunchKernelGGL((q4_gemv_kernel<NGB, 2, XS, TAIL, XL, BF, W8, MB, R1>), dim3((p.N + 31) / 32, splits), block, lds, stream, Q4_GEMV_ARGS(p)); break;
    case 4:
        // (8-bit blocks are twice the registers: at most two tiles)
        if constexpr (W8) return hipErrorInvalidValue;
        else hipLaunchKernelGGL((q4_gemv_kernel<NGB, 4, XS, TAIL, XL, BF, W8, MB, R1>), dim3((p.N + 63) / 64, splits), block, lds, stream, Q4_GEMV_ARGS(p));
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Activation loads: one per 4 k-steps for M <= 4, per 2 for M <= 8, else one
// per k-step. A K that is not a multiple of 128 (one partial block) takes the
// one-per-step form, whose past-K steps are masked per load. M > 16 takes
// two row blocks of 16, one load per k-step each.
// (Staged act-order activations come with M <= 2 only.)
template <int NGB, bool XL, bool BF, bool W8>
hipError_t launch_ngb(const GemvArgs& p, int ct, int splits, hipStream_t stream)
{
    if constexpr (!XL) {
        if (p.M > 16) {
            return p.K % 128 != 0 ? launch_ct<NGB, 1, true, false, BF, W8, 2>(p, ct, splits, stream)
                                  : launch_ct<NGB, 1, false, false, BF, W8, 2>(p, ct, splits, stream);
        }
    }
    if (p.K % 128) return launch_ct<NGB, 1, true, XL, BF, W8, 1>(p, ct, splits, stream);
    if (p.M == 1) return launch_ct<NGB, 4, false, XL, BF, W8, 1, true>(p, ct, splits, stream);
    if (p.M <= 4 || XL) return launch_ct<NGB, 4, false, XL, BF, W8, 1>(p, ct, splits, stream);
    if constexpr (!XL) {
        if (p.M <= 8) return launch_ct<NGB, 2, false, XL, BF, W8, 1>(p, ct, splits, stream);
        return launch_ct<NGB, 1, false, XL, BF, W8, 1>(p, ct, splits, stream);
    }
    return hipErrorInvalidValue;
}

template <bool XL, bool BF, bool W8>
hipError_t launch_xl(const GemvArgs& p, int ngb, int ct, int splits, hipStream_t stream)
{
    switch (ngb) {
    case 1: return launch_ngb<1, XL, BF, W8>(p, ct, splits, stream);
    case 2: return launch_ngb<2, XL, BF, W8>(p, ct, splits, stream);
    case 4: return launch_ngb<4, XL, BF, W8>(p, ct, splits, stream);
    default: return hipErrorInvalidValue;
    }
}

template <bool W8>
hipError_t launch_w(const GemvArgs& p, int ngb, int ct, int splits, bool gather_x, bool bf16,
                    hipStream_t stream)
{
    if (bf16)
        return gather_x ? launch_xl<true, true, W8>(p, ngb, ct, splits, stream)
                        : launch_xl<false, true, W8>(p, ngb, ct, splits, stream);
    return gather_x ? launch_xl<true, false, W8>(p, ngb, ct, splits, stream)
                    : launch_xl<false, false, W8>(p, ngb, ct, splits, stream);
}

}  // namespace

namespace q4 {

hipError_t launch_gemv(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
                       int M, int col_tiles, int splits, bool gather_x, bool bf16, float* partials,
                       uint32_t* counters, hipStream_t stream)
{
    if (M < 1 || M > kGemvMaxM || splits < 1 || splits > kMaxSplits) return hipErrorInvalidValue;
    if (splits > 1 && (!partials || !counters)) return hipErrorInvalidValue;
    if (M > 16 && gather_x) return hipErrorInvalidValue;
    if (gather_x && (!h->inv16 || !gemv_gathers_x(M, h->K, splits))) return hipErrorInvalidValue;
    GemvArgs p;
    p.qweight = h->qweight;
    p.sz = h->sz;
    p.x = x;
    p.inv = gather_x ? h->inv16 : nullptr;
    p.bias = bias;
    p.out = out;
    p.partials = partials;
    p.counters = counters;
    p.M = M;
    p.K = h->K;
    p.N = h->N;
    p.G = h->G;
    p.ng = h->ng;
    // k-steps (32 rows) per group = 2^gshift; one group over K never changes
    p.gshift = 31;
    if (h->G != h->K)
        for (int sh = 0; sh < 4; ++sh)
            if ((32 << sh) == h->G) p.gshift = sh;
    p.kblocks = num_kblocks(h->K);
    p.splits = splits;
    p.blocks_per_split = (p.kblocks + splits - 1) / splits;
    p.blocks_per_wave = (p.blocks_per_split + kGemvWaves - 1) / kGemvWaves;
    p.ldx = gather_x ? p.kblocks * 128 + kGemvXPad : 0;
    // groups per 128-row block: groups of 32 or 64 rows split a block; larger
    // groups (and one group over K) cover it whole
    const int ngb = (h->G == h->K || h->G >= 128) ? 1 : 128 / h->G;
    return h->bits == 8 ? launch_w<true>(p, ngb, col_tiles, splits, gather_x, bf16, stream)
                        : launch_w<false>(p, ngb, col_tiles, splits, gather_x, bf16, stream);
}

}  // namespace q4
