// Prefill fused GPTQ GEMM (M > 16) on the matrix cores: activations staged
// in LDS, weights streamed into registers.
//
// q4_gemm_stream_kernel<BM, NG, KT, BF, W8>: BM rows per output tile (256,
// or 64 when M <= 512), NG groups per 64-row k-tile (2 for groups of 32), KT
// (K not a multiple of 64), BF (bfloat16 activations and output), W8 (8-bit
// codes).
//
// The multiply runs on v_mfma_f32_32x32x16_f16 with fp32 accumulation
// (GPTQModel wiki "Inference Backends", hardware table, ExLlama v2 row: FP32
// accumulation, FP16 scales). The packed weights never touch LDS: every wave
// loads the words of its own columns straight into registers, one k-tile
// ahead, and dequantizes them there for the MFMA, so no dequantized weight
// exists anywhere but in registers ("GPTQ's 'Exllama Kernel Not Installed'
// Warning", section "What the fallback actually does").
//
// Tiling: a workgroup of 4 waves computes a BM x 128 output tile; each wave
// owns BM x 32 (BM / 32 MFMA tiles of 32 x 32, one column tile). K advances
// in 64-row tiles.
//  * Activations: a 2-stage LDS ring (32 KiB a stage, 16-byte chunks of the
//    128-byte rows XOR-swizzled by (row / 2) % 8) filled by direct-to-LDS
//    buffer loads. 64 KiB of LDS lets two workgroups share a CU.
//  * Weights: for its column (lane % 32 of the wave's 32) a lane needs, per k-tile, words 2h and
//    2h + 1 of chunks (b, kb) and (b, kb + 2) of the private block layout
//    (k-tile 2b + h, kb = lane / 32): two 8-byte loads. With the
//    32-bit scale|zero word of each of the tile's groups (built by the make
//    step, as for the skinny kernel), these go to one of two register sets;
//    the k-loop is unrolled by two so that the set a step multiplies is never
//    a set a load is filling.
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
#include "q4_fastdiv.h"
#include "q4_internal.h"

namespace {

using namespace q4dev;

constexpr int BK = q4::kGemmBK;      // 64
// The NW waves of a workgroup sit side by side along N (1 x NW): each owns
// all BM rows of 32 columns, so every packed word is dequantized by exactly
// one wave and each wave reads the whole activation stage from LDS. (A 2 x 2
// grid of four waves reads half the activations per wave but dequantizes
// every word twice; measured slower: M = 2048 948 -> 969 TFLOP/s on
// 4096x11008, M = 256 453 -> 601, M = 64 264 -> 291. LDS reads stay under a
// third of the LDS bandwidth.) NW = 4 (128-column tiles, two workgroups per
// CU) or 8 (256-column tiles, one per CU: the activation stage each copies
// from L2 serves twice the columns).
constexpr int NJ = 1;                // 32-column MFMA tiles per wave
static_assert(BK == 64, "index arithmetic below assumes 64-row k-tiles");

// Geometry that depends on the tile height BM (256, or 64 for few rows) and
// the waves NW: each wave owns BM x 32 (MI MFMA tiles of 32 x 32); the
// activation stage is BM x BK halfs, filled by A_LOADS 16-byte direct loads
// per thread (BM = 256: 8 with four waves, 4 with eight; 32 KiB a stage;
// BM = 64: 2 with four waves, 8 KiB).
template <int BM, int NW>
struct Geo {
    static constexpr int NT = 64 * NW;
    static constexpr int BN = 32 * NW;
    static constexpr int MI = BM / 32;
    static constexpr int A_TILE_BYTES = BM * BK * 2;
    static constexpr int A_LOADS = A_TILE_BYTES / (NT * 16);
    static_assert((NW == 4 || NW == 8) && MI >= 1 && A_LOADS >= 1 && A_TILE_BYTES == A_LOADS * NT * 16,
                  "tile shape");
};

typedef __attribute__((address_space(3))) void lds_void;

struct GemmArgs {
    const uint32_t* qweight;
    const uint32_t* sz;     // [ng][N]: scale bits | zero point << 16
    const uint16_t* x;
    const uint16_t* bias;
    uint16_t* out;
    int M, K, N, G;
    int gshift;             // group of row k = k >> gshift (31: one group over K)
    // Schedule: `workers` workgroups share the (output tile, k-tile)
    // iterations evenly, in contiguous ranges, each at least one iteration
    // long (workers <= iterations). workers = tiles is one tile per
    // workgroup; fewer or more split some tiles' K ranges between workgroups
    // (stream-K), whose fp32 partial sums go through `partials` (two
    // 256 x 128 slots per workgroup) and an arrival counter per split tile
    // (zero between launches).
    float* partials;
    uint32_t* counters;
    int workers;
    int xcd;                // 1: each XCD takes the row tiles r with r % 8 == XCD (row tiles % 8 == 0)
    // The same split in 32-bit terms, set by the host (iterations < 2^30):
    // a space of `iters` iterations shared by `ps` workgroups, with
    // iters = iq * ps + ir; k-tiles per output tile and column tiles; and
    // multipliers for dividing by ps, ktiles and nt.
    uint32_t iters, ps, iq, ir, ktiles, nt;
    q4::FastDiv div_ps, div_kt, div_nt;
    float ps_per_iter;      // ps / iters (the owner estimate below)
};

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>), unrolled
template <int I, int N, class F>
__device__ __forceinline__ void static_for_from(F&& f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_from<I + 1, N>(f);
    }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) { static_for_from<0, N>(f); }

__device__ __forceinline__ uint32_t swz(int r, int c) { return (uint32_t)(r * 128 + ((c ^ ((r >> 1) & 7)) << 4)); }

#define Q4S_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One k-tile of a lane's weights: w[j][0] = words (2h, 2h+1) of chunk
// (b, kb, n_j) -- sub-steps 0 and 2 -- and w[j][1] those of chunk
// (b, kb + 2, n_j) -- sub-steps 1 and 3; the scale|zero words of the tile's
// NG groups (two for groups of 32 rows).
template <int NG, bool W8>
struct BRegs {
    std::conditional_t<W8, u4, u2> w[NJ][2];
    uint32_t sz[NG][NJ];    // scale bits | zero point << 16
};

constexpr int kMaxALoads = Geo<256, 4>::A_LOADS;
struct Ctx {
    rsrc_t rx, rw, rsz;
    // (the first A_LOADS entries are used)
    uint32_t a_off[kMaxALoads];   // activation byte offsets for k0 = 0 (rows >= M fall outside x)
    uint32_t a_k[kMaxALoads];     // k of each chunk for k0 = 0
    uint32_t w_off[NJ][2];     // weight byte offsets of the two chunks per column (k-tile 0)
    uint32_t sz_off[NJ];       // group-word byte offsets (group 0)
};

// The k offset of the tile is wave-uniform (a scalar register); rows past M
// lie past the end of x through the per-lane offset alone. Only with KT can a
// chunk lie past K (in the last tile); its lanes are pushed out of range.
template <bool KT, int A_LOADS, int NW>
__device__ __forceinline__ void load_a(const Ctx& c, const GemmArgs& p, char* stage, int wave, int kt)
{
    const uint32_t k0 = (uint32_t)kt * BK;
#pragma unroll
    for (int e = 0; e < A_LOADS; ++e) {
        const uint32_t kill = (!KT || c.a_k[e] + k0 < (uint32_t)p.K) ? 0u : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rx, (lds_void*)(stage + (e * NW + wave) * 1024), 16,
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
        const uint32_t g = (uint32_t)k >> p.gshift;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            R.sz[gi][j] = buf_load4(c.rsz, c.sz_off[j], g * (uint32_t)p.N * 4u);
        }
    }
}

// KT: K is not a multiple of 64, so the last k-tile skips its sub-steps past
// K (a separate instantiation, so that the common kernel has no branch
// around the multiply: the accumulators stay in the same registers).
// (Two workgroups per CU: the register budget is 256 per lane.)
template <int BM, int NW, int NG, bool KT, bool BF, bool W8>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void q4_gemm_stream_kernel(GemmArgs p)
{
    using G = Geo<BM, NW>;
    constexpr int NT = G::NT, BN = G::BN, MI = G::MI, WTM = BM;
    constexpr int A_TILE_BYTES = G::A_TILE_BYTES, A_LOADS = G::A_LOADS;
    // Ring depth: activation stages in LDS and weight register sets, both
    // D - 1 k-tiles ahead: three for 64-row tiles (few rows), two for the
    // 256-row, 256-column tiles (96 KiB of LDS, one workgroup per CU), one
    // for 256-row, 128-column tiles (two workgroups per CU share 160 KiB).
    // (Deeper 64-row rings first measured slower: the compiler then reused a
    // few registers for the activation reads and waited out one LDS latency
    // per sub-step. With all reads of a k-tile issued together (mma below),
    // four stages beat three by 2-9% at M = 33 ... 128 on the 7B MLP shapes
    // and 4096 x 4096.)
    constexpr int D = BM == 64 ? 4 : NW == 8 ? 3 : 2;
    // vector-memory loads one step issues per thread (activation DMA, packed
    // weights, scale|zero words)
    constexpr int LPS = A_LOADS + 2 * NJ + NG * NJ;
    // One array per stage: the compiler tells the stages apart by their
    // variables, so reading one stage does not wait for the direct-to-LDS
    // loads into another (with one array of stages it waits for them all).
    static_assert(D >= 2 && D <= 8, "ring depth");
    __shared__ __attribute__((aligned(1024))) char lds_a0[A_TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_a1[A_TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char lds_a2[D > 2 ? A_TILE_BYTES : 1];
    __shared__ __attribute__((aligned(1024))) char lds_a3[D > 3 ? A_TILE_BYTES : 1];
    __shared__ __attribute__((aligned(1024))) char lds_a4[D > 4 ? A_TILE_BYTES : 1];
    __shared__ __attribute__((aligned(1024))) char lds_a5[D > 5 ? A_TILE_BYTES : 1];
    __shared__ __attribute__((aligned(1024))) char lds_a6[D > 6 ? A_TILE_BYTES : 1];
    __shared__ __attribute__((aligned(1024))) char lds_a7[D > 7 ? A_TILE_BYTES : 1];
    __shared__ int s_last;

    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int wm = 0, wn = wave;   // (waves side by side along N)
    // per-lane indices, recomputed for every segment (below) so that values
    // derived from them are not kept live across the k-loop
    int tid = 0, lane = 0, l32 = 0, lhi = 0;

    // Iteration space. With `xcd`, workgroup i runs on XCD i % 8 and works on
    // that XCD's own row tiles (row tile r with r % 8 == XCD), which keeps
    // their activations in its L2; otherwise one space in row-major tile
    // order. A space of T tiles holds T * ktiles iterations (tile-major);
    // worker r of Ps takes iterations [r * I / Ps, (r + 1) * I / Ps).
    // (All of this is wave-uniform 32-bit arithmetic: 64-bit divisions here
    // compiled to about 1200 scalar instructions, 1.1 us before the first
    // load of every workgroup.)
    const uint32_t ktiles = p.ktiles, nt = p.nt;
    const int id = blockIdx.x;
    const int space = p.xcd ? (id & 7) : 0;
    const int rk = p.xcd ? (id >> 3) : id;
    // first iteration of worker r: floor(r * iters / ps) = r * iq + floor(r * ir / ps)
    auto begin_of = [&](int r) { return (uint32_t)r * p.iq + q4::fast_div((uint32_t)r * p.ir, p.div_ps); };
    const uint32_t it_begin = begin_of(rk), it_end = begin_of(rk + 1);
    // worker of iteration i: the largest r with begin_of(r) <= i (a float
    // estimate, off by at most one or two, then corrected)
    auto owner = [&](uint32_t i) {
        int r = min((int)((float)i * p.ps_per_iter), (int)p.ps - 1);
        while (r > 0 && begin_of(r) > i) --r;
        while (r + 1 < (int)p.ps && begin_of(r + 1) <= i) ++r;
        return r;
    };
    auto worker_id = [&](int r) { return p.xcd ? r * 8 + space : r; };

    Ctx c;
    const int ng = p.K / p.G;
    c.rx = make_rsrc(p.x, (uint32_t)p.M * (uint32_t)p.K * 2u);
    c.rw = make_rsrc(p.qweight, (uint32_t)q4::num_kblocks(p.K) * (uint32_t)p.N * (W8 ? 128u : 64u));
    c.rsz = make_rsrc(p.sz, (uint32_t)ng * (uint32_t)p.N * 4u);

    f16x acc[MI][NJ];
    BRegs<NG, W8> R[D];
    // the unpack's OR constant in a register (see and_or)
    uint32_t magic = kMagic2;
    asm volatile("" : "+v"(magic));
    int m0 = 0, seg_end = 0;
    int lane_cols[NJ];
    // Whether row group g (rows 8g .. 8g + 7) of MFMA row tile i of the
    // current output tile has a row below M, a wave-uniform test: accumulator
    // registers r with r / 4 == g hold those rows (in lane halves 0 and 1).
    auto row_group_in = [&](int i, int g) { return m0 + 32 * i + 8 * g < p.M; };

    // Multiply k-tile kt: activations from `A`, weights from register set R.
    // Software-pipelined over the four 16-row sub-steps: the weights of
    // sub-step s + 1 are dequantized while the eight MFMAs of sub-step s run,
    // and the scheduling groups below interleave those vector instructions
    // with the MFMAs (the matrix pipe takes 32 cycles per MFMA, during which
    // the wave can issue independent vector instructions) instead of leaving
    // a burst of dequantization ahead of each sub-step's MFMAs.
    // With KT, sub-steps past K (zero activations) are skipped so that their
    // weights (code 0, any scale) add nothing.
    auto mma = [&](const char* A, const BRegs<NG, W8>& R, int kt) {
        zero_t hz[NG][NJ];
        h2 s2[NG][NJ];
        mix_t mz[NJ];   // BF: the constants of the group being dequantized (registers)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if constexpr (!BF) {
                    hz[gi][j] = zero_pair_sz(R.sz[gi][j], magic);
                    s2[gi][j] = scale_pair(R.sz[gi][j]);
                }
            }
        // dequantize sub-step `sub` of this k-tile into b
        auto deq = [&](int sub, u4 (&b)[NJ]) {
            const int gi = NG == 2 ? (sub >> 1) : 0;
            if constexpr (BF) {
                if (sub % (4 / NG) == 0)
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
                        mz[j] = mix_consts(R.sz[gi][j] >> 16, f16_bits_to_f32((uint16_t)R.sz[gi][j]), magic);
            }
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
        };
        const int k0 = kt * BK;
        u4 bc[NJ], bn[NJ];
        auto read_a = [&](int sub, int i) {
            return *reinterpret_cast<const u4*>(A + swz(wm * WTM + 32 * i + l32, 2 * sub + lhi));
        };
        if constexpr (MI <= 2) {
            // Few rows: one wave per SIMD, so nothing else hides a read's
            // latency. The whole k-tile's activations are read at once, and
            // each sub-step's MFMAs are interleaved with the dequantization
            // of the next sub-step's weights.
            u4 aa[BK / 16][MI];
#pragma unroll
            for (int sub = 0; sub < BK / 16; ++sub)
#pragma unroll
                for (int i = 0; i < MI; ++i) aa[sub][i] = read_a(sub, i);
            // (all of them issued before the first MFMA: otherwise the
            // compiler reuses a few registers for them and waits out one
            // LDS latency per sub-step)
            __builtin_amdgcn_sched_group_barrier(0x100, BK / 16 * MI, 0);
            deq(0, bc);
#pragma unroll
            for (int sub = 0; sub < BK / 16; ++sub) {
                if (sub + 1 < BK / 16) deq(sub + 1, bn);
                const bool live = !KT || k0 + 16 * sub < p.K;
                if (live) {
#pragma unroll
                    for (int i = 0; i < MI; ++i)
#pragma unroll
                        for (int j = 0; j < NJ; ++j) {
                            if constexpr (BF) acc[i][j] = mfma32(bitcast<b8>(aa[sub][i]), bitcast<b8>(bc[j]), acc[i][j]);
                            else acc[i][j] = mfma32(bitcast<h8>(aa[sub][i]), bitcast<h8>(bc[j]), acc[i][j]);
                        }
                }
                if (sub + 1 < BK / 16) {
#pragma unroll
                    for (int q = 0; q < MI * NJ; ++q) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
                    }
                }
#pragma unroll
                for (int j = 0; j < NJ; ++j) bc[j] = bn[j];
            }
            return;
        }
        u4 a[MI];
#pragma unroll
        for (int i = 0; i < MI; ++i) a[i] = read_a(0, i);
        deq(0, bc);
#pragma unroll
        for (int sub = 0; sub < BK / 16; ++sub) {
            if (sub + 1 < BK / 16) deq(sub + 1, bn);
            const bool live = !KT || k0 + 16 * sub < p.K;
            // row tile i's MFMAs, then its activations for the next
            // sub-step into the same registers
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                if (live) {
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        if constexpr (BF) acc[i][j] = mfma32(bitcast<b8>(a[i]), bitcast<b8>(bc[j]), acc[i][j]);
                        else acc[i][j] = mfma32(bitcast<h8>(a[i]), bitcast<h8>(bc[j]), acc[i][j]);
                    }
                }
                if (sub + 1 < BK / 16) a[i] = read_a(sub + 1, i);
            }
            if (sub + 1 < BK / 16) {
                // each MFMA followed by one activation read and up to two
                // vector instructions of the next sub-step
#pragma unroll
                for (int q = 0; q < MI * NJ; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (q < MI) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                }
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) bc[j] = bn[j];
        }
    };

    auto stage = [&](int st) -> char* {
        switch (st) {
        case 0: return lds_a0;
        case 1: return lds_a1;
        case 2: return lds_a2;
        case 3: return lds_a3;
        case 4: return lds_a4;
        case 5: return lds_a5;
        case 6: return lds_a6;
        default: return lds_a7;
        }
    };

    // One k-tile on stage and register set S = (kt - segment start) % D,
    // prefetching tile kt + D - 1 (clamped: past the segment's end it
    // reloads its last tile, into buffers nobody reads again) into the stage
    // and set tile kt - 1 has just finished with.
    auto step = [&](auto S_tag, int kt) {
        constexpr int S = decltype(S_tag)::value;
        constexpr int SN = (S + D - 1) % D;
        // Tile kt's activations and weight registers must have landed (the
        // activations in every thread's part of the stage). The D - 2 steps
        // since its loads each issued LPS loads, and scheduling barriers keep
        // every step's loads inside that step, so the count holds whatever
        // order a step issues its own loads in (D = 2: no count at all).
        Q4S_VMCNT((D - 2) * LPS);
        lds_barrier();
        const int kn = min(kt + D - 1, seg_end - 1);
        if constexpr (D > 2) __builtin_amdgcn_sched_barrier(0);
        load_a<KT, A_LOADS, NW>(c, p, stage(SN), wave, kn);
        load_b(R[SN], c, p, kn);
        // (with D = 2 the wait above counts nothing, and leaving the loads
        // free to move measured 1-2% faster)
        if constexpr (D > 2) __builtin_amdgcn_sched_barrier(0);
        mma(stage(S), R[S], kt);
    };

    // The range [a, b) is the tail of a split tile [a, lo), whole tiles
    // [lo, hi) and the head of a split tile [hi, b). The two split segments
    // go first: the neighbouring workgroups also start with theirs, so both
    // halves of a split tile finish early and its fix-up overlaps the whole
    // tiles of this workgroup and of the one sharing its CU, instead of all
    // fix-ups landing at the end of the kernel.
    const uint32_t lo = min(it_end, q4::fast_div(it_begin + ktiles - 1, p.div_kt) * ktiles);
    const uint32_t hi = max(lo, q4::fast_div(it_end, p.div_kt) * ktiles);
    const int nfull = (int)q4::fast_div(hi - lo, p.div_kt);
    bool first_seg = true;
    for (int sg = -2; sg < nfull; ++sg) {
        const uint32_t sb = sg == -2 ? it_begin : sg == -1 ? hi : lo + (uint32_t)sg * ktiles;
        const uint32_t se = sg == -2 ? lo : sg == -1 ? it_end : sb + ktiles;
        if (sb >= se) continue;
        const uint32_t lt = q4::fast_div(sb, p.div_kt);
        const int kb = (int)(sb - lt * ktiles);
        const int ke = kb + (int)(se - sb);
        const uint32_t tr = q4::fast_div(lt, p.div_nt);   // row tile within the space
        const int mtile = p.xcd ? (int)tr * 8 + space : (int)tr;
        const int n0 = (int)(lt - tr * nt) * BN;
        m0 = mtile * BM;
        seg_end = ke;
        tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        lane = tid & 63;
        l32 = lane & 31;
        lhi = lane >> 5;
#pragma unroll
        for (int e = 0; e < A_LOADS; ++e) {
            // instruction e of wave w fills rows 8 * (4e + w) .. +7 of the stage;
            // lane i lands in slot i % 8 of row i / 8, which holds chunk
            // slot ^ ((row >> 1) & 7)
            const int row = 8 * (NW * e + wave) + (lane >> 3);
            const int chunk = (lane & 7) ^ ((row >> 1) & 7);
            c.a_k[e] = 8u * (uint32_t)chunk;
            c.a_off[e] = ((uint32_t)(m0 + row) * (uint32_t)p.K + c.a_k[e]) * 2u;
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            lane_cols[j] = n0 + wn * 32 + 32 * j + l32;
            const uint32_t n = (uint32_t)min(lane_cols[j], p.N - 1);   // columns past N are never stored
#pragma unroll
            for (int v = 0; v < 2; ++v) c.w_off[j][v] = q4::chunk_in_block(lhi + 2 * v, (int)n, p.N) * (W8 ? 32u : 16u);
            c.sz_off[j] = n * 4u;
        }
        // the bias of the lane's columns, loaded before the k-loop so that
        // its latency hides behind it (the loop's counted waits then also
        // cover this oldest load, which only makes the first wait exact)
        uint16_t bias_h[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) bias_h[j] = p.bias ? p.bias[min(lane_cols[j], p.N - 1)] : (uint16_t)0;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

        // Every wave has finished reading the stages (previous segment)
        // before they are refilled.
        if (!first_seg) lds_barrier();
        first_seg = false;
#pragma unroll
        for (int d = 0; d + 1 < D; ++d) {
            const int kd = min(kb + d, ke - 1);
            load_a<KT, A_LOADS, NW>(c, p, stage(d), wave, kd);
            load_b(R[d], c, p, kd);
            if constexpr (D > 2) __builtin_amdgcn_sched_barrier(0);
        }
        int kt = kb;
        for (; kt + D - 1 < ke; kt += D)
            static_for<D>([&](auto S_tag) { step(S_tag, kt + decltype(S_tag)::value); });
        // the last 0 .. D - 1 tiles
        static_for<D - 1>([&](auto S_tag) {
            if (kt + decltype(S_tag)::value < ke) step(S_tag, kt + decltype(S_tag)::value);
        });
        // Drain the last (unused) prefetch before the LDS is reused.
        Q4S_VMCNT(0);

        if (kb != 0 || ke != (int)ktiles) {
            // A split tile, whose workers wf .. wl each hold one k-segment.
            // The last of them to arrive adds the fp32 sums in k order,
            // p_wf + p_wf+1 + ... + p_wl (the same bits whichever worker that
            // is), and stores. The others publish their sums first: agent-
            // scope atomic stores and loads go to the device-coherent level
            // (a full fence would write back and invalidate the XCD's L2),
            // and every wave's stores are complete before the arrival count
            // is bumped. A worker that finds all the others already counted
            // is last without publishing its own.
            // Slots: a segment that starts inside its tile is its worker's
            // first (slot 2 id), one that starts the tile is its worker's
            // last (slot 2 id + 1).
            const uint32_t t0 = lt * ktiles;
            const int wf = owner(t0), wl = owner(t0 + ktiles - 1);
            const uint32_t others = (uint32_t)(wl - wf);
            auto slot_of = [&](int r) {
                return p.partials + (size_t)(r == wf ? 2 * worker_id(r) + 1 : 2 * worker_id(r)) * (BM * BN);
            };
            uint32_t* counter = p.counters + worker_id(wf);
            // (Reading the arrival count while the sums go out, rather than
            // first, measured 4% slower on the 256-row tiles of 4096 x 11008:
            // a last worker then publishes 128 KiB that nobody reads.)
            if (tid == 0)
                s_last = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == others;
            __syncthreads();
            if (!s_last) {
                float* mine = slot_of(rk);
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < NJ; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            __hip_atomic_store(&mine[((i * NJ + j) * 16 + r) * NT + tid], acc[i][j][r],
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (tid == 0)
                    s_last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                             others;
                __syncthreads();
                if (!s_last) continue;
            }
            // Ordered sum, 32 values per lane at a time: p_wf + ... + p_wl,
            // this worker's own sums taken from its registers. With 64-row
            // tiles (up to eight contributors on a narrow layer) the other
            // workers' slots are read FB at a time, all loads of a batch in
            // flight together: 1-2% faster at M = 33 ... 256 than one worker
            // at a time (these loads are bound more by the rate at which one
            // CU fetches device-coherent data than by their latency). 256-row
            // tiles keep one at a time: their accumulators leave no room.
            constexpr int FB = MI <= 2 ? 4 : 1;
            auto load32 = [&](float (&v)[32], int r, int q) {
                const float* src = slot_of(r) + (size_t)q * 16 * NT + tid;
#pragma unroll
                for (int e = 0; e < 32; ++e)
                    v[e] = __hip_atomic_load(&src[e * NT], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            };
            // workers r0 .. r1 in batches of FB; f(v, r) consumes worker r's
            // values, in worker order
            auto batches = [&](int r0, int r1, int q, auto&& f) {
                for (int rb = r0; rb <= r1; rb += FB) {
                    float v[FB][32];
#pragma unroll
                    for (int b = 0; b < FB; ++b)
                        if (rb + b <= r1) load32(v[b], rb + b, q);
#pragma unroll
                    for (int b = 0; b < FB; ++b)
                        if (rb + b <= r1) f(v[b], rb + b);
                }
            };
#pragma unroll
            for (int q = 0; q < MI * NJ; q += 2) {
#define Q4S_ACC(e) acc[(q + (e) / 16) / NJ][(q + (e) / 16) % NJ][(e) % 16]
                if (rk > wf) {
                    // p_wf + ... + p_(rk-1), then + this worker's sums
                    float t[32];
                    batches(wf, rk - 1, q, [&](const float (&v)[32], int r) {
#pragma unroll
                        for (int e = 0; e < 32; ++e) t[e] = r == wf ? v[e] : t[e] + v[e];
                    });
#pragma unroll
                    for (int e = 0; e < 32; ++e) Q4S_ACC(e) = t[e] + Q4S_ACC(e);
                }
                batches(rk + 1, wl, q, [&](const float (&v)[32], int) {
#pragma unroll
                    for (int e = 0; e < 32; ++e) Q4S_ACC(e) += v[e];
                });
#undef Q4S_ACC
            }
            if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        // Epilogue: fp32 bias, one round-to-nearest-even cast, store. Lane l
        // holds rows 8*(r/4) + 4*(l/32) + r%4 of column l%32 of each 32 x 32
        // tile. A whole row tile stores through a buffer descriptor, the row
        // part of each offset wave-uniform, with no per-element checks (a
        // compare and branch per element cost about 1 us of a 64-row tile's
        // epilogue); a partial row tile uses the descriptor's range instead
        // (below).
        const rsrc_t ro = make_rsrc(p.out, (uint32_t)p.M * (uint32_t)p.N * 2u);
        const bool whole = m0 + BM <= p.M;
        // A partial row tile stores through the same descriptor with the
        // whole offset per lane, skipping the row groups that lie past M: a
        // store to a row past M then lies past the descriptor's end, which
        // drops it. Those rows are below M + 8, so their offsets stay under
        // 2^32 unless (M + 8) N * 2 does not (then each element is checked).
        const bool ranged = !whole && (uint64_t)(p.M + 8) * (uint64_t)p.N * 2u < (1ull << 32);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int n = lane_cols[j];
            if (n >= p.N) continue;
            // (the conversion stays here: left to the compiler it moves up to
            // the load and waits for it before the k-loop)
            uint32_t bh = bias_h[j];
            asm volatile("" : "+v"(bh));
            const float bv = p.bias ? act_to_f32<BF>((uint16_t)bh) : 0.f;
            const int mb = m0 + wm * WTM + 4 * lhi;   // the lane's first row
            if (whole) {
                // (m * N + n) * 2 < M * N * 2 <= 2^32 - 2: no wrap-around
                const uint32_t voff = ((uint32_t)mb * (uint32_t)p.N + (uint32_t)n) * 2u;
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const uint32_t dr = (uint32_t)(32 * i + 8 * (r >> 2) + (r & 3));
                        buf_store2(ro, voff, dr * (uint32_t)p.N * 2u, f32_to_act<BF>(acc[i][j][r] + bv));
                    }
            } else if (ranged) {
                const uint32_t voff = ((uint32_t)mb * (uint32_t)p.N + (uint32_t)n) * 2u;
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        if (!row_group_in(i, r >> 2)) continue;
                        const uint32_t dr = (uint32_t)(32 * i + 8 * (r >> 2) + (r & 3));
                        buf_store2(ro, voff + dr * (uint32_t)p.N * 2u, 0u, f32_to_act<BF>(acc[i][j][r] + bv));
                    }
            } else {
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = mb + 32 * i + 8 * (r >> 2) + (r & 3);
                        if (m < p.M) p.out[(size_t)m * p.N + n] = f32_to_act<BF>(acc[i][j][r] + bv);
                    }
            }
        }
    }
}

template <int BM, int NW, bool BF, bool W8>
hipError_t launch_stream(const GemmArgs& p, int grid, bool g32, bool kt, hipStream_t stream)
{
    const dim3 block(64 * NW);
    if (g32 && kt)
        hipLaunchKernelGGL((q4_gemm_stream_kernel<BM, NW, 2, true, BF, W8>), dim3(grid), block, 0, stream, p);
    else if (g32)
        hipLaunchKernelGGL((q4_gemm_stream_kernel<BM, NW, 2, false, BF, W8>), dim3(grid), block, 0, stream, p);
    else if (kt)
        hipLaunchKernelGGL((q4_gemm_stream_kernel<BM, NW, 1, true, BF, W8>), dim3(grid), block, 0, stream, p);
    else
        hipLaunchKernelGGL((q4_gemm_stream_kernel<BM, NW, 1, false, BF, W8>), dim3(grid), block, 0, stream, p);
    return hipGetLastError();
}

template <int BM, int NW>
hipError_t launch_bm(const GemmArgs& p, int grid, bool g32, bool kt, bool bf16, bool w8, hipStream_t stream)
{
    if (w8)
        return bf16 ? launch_stream<BM, NW, true, true>(p, grid, g32, kt, stream)
                    : launch_stream<BM, NW, false, true>(p, grid, g32, kt, stream);
    return bf16 ? launch_stream<BM, NW, true, false>(p, grid, g32, kt, stream)
                : launch_stream<BM, NW, false, false>(p, grid, g32, kt, stream);
}

}  // namespace

namespace q4 {

hipError_t launch_gemm_stream(const q4_matrix* h, const uint16_t* x, const uint16_t* bias, uint16_t* out,
                              int M, bool bf16, int waves, int workers, float* partials, uint32_t* counters,
                              hipStream_t stream)
{
    // 256-column tiles (eight waves) only with 256-row tiles
    const int bm = gemm_bm(M);
    if (waves != 4 && !(waves == 8 && bm == kGemmBM)) return hipErrorInvalidValue;
    const int BN = 32 * waves;
    GemmArgs p;
    p.qweight = h->qweight;
    p.sz = h->sz;
    p.x = x;
    p.bias = bias;
    p.out = out;
    p.M = M;
    p.K = h->K;
    p.N = h->N;
    p.G = h->G;
    // groups are 32, 64, 128 or 256 rows, or one group over K
    p.gshift = 31;
    if (h->G != h->K)
        for (int sh = 5; sh <= 8; ++sh)
            if ((1 << sh) == h->G) p.gshift = sh;
    p.partials = partials;
    p.counters = counters;
    p.workers = workers;
    // XCD spaces need whole row tiles and workers per XCD
    const uint32_t mt = (uint32_t)((M + bm - 1) / bm), nt = (uint32_t)((h->N + BN - 1) / BN);
    const uint32_t ktiles = (uint32_t)((h->K + BK - 1) / BK);
    p.xcd = mt % 8 == 0 && workers % 8 == 0;
    const uint64_t iters = (uint64_t)(p.xcd ? mt / 8 : mt) * nt * ktiles;
    const uint32_t ps = (uint32_t)(p.xcd ? workers / 8 : workers);
    // (matmul_impl rejects larger products with a message; the kernel's
    // index arithmetic is 32-bit)
    if (workers < 1 || iters >= (1u << 30) || ps > iters) return hipErrorInvalidValue;
    p.iters = (uint32_t)iters;
    p.ps = ps;
    p.iq = p.iters / ps;
    p.ir = p.iters % ps;
    p.ktiles = ktiles;
    p.nt = nt;
    p.div_ps = make_fastdiv(ps);
    p.div_kt = make_fastdiv(ktiles);
    p.div_nt = make_fastdiv(nt);
    p.ps_per_iter = (float)ps / (float)p.iters;
    // Groups of 64 rows or more never straddle a 64-row k-tile; groups of 32
    // change once inside it.
    const bool g32 = h->G % BK != 0 && h->G != h->K, kt = h->K % BK != 0;
    if (bm == 64) return launch_bm<64, 4>(p, workers, g32, kt, bf16, h->bits == 8, stream);
    return waves == 8 ? launch_bm<kGemmBM, 8>(p, workers, g32, kt, bf16, h->bits == 8, stream)
                      : launch_bm<kGemmBM, 4>(p, workers, g32, kt, bf16, h->bits == 8, stream);
}

}  // namespace q4
