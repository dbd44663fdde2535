// Device-side helpers shared by the libq4 kernels: the in-register unpack and
// dequantization of one packed 32-bit word, and MFMA operand types.
//
// Dequantization ("GPTQ's 'Exllama Kernel Not Installed' Warning", section
// "What the fallback actually does": the fused kernel unpacks and dequantizes
// in registers) produces, for each 4-bit code q with zero point z and fp16
// scale s, the binary16 value RNE(s * (q - z)):
//
//  * binary16 0x6400 is 1024.0 (biased exponent 25) and its fraction ulp is
//    1, so OR-ing a code into fraction bits 0..3 yields exactly 1024 + q;
//  * (1024 + q) - (1024 + z) = q - z is exact in fp16 (|q - z| <= 15);
//  * the fp16 product (q - z) * s is the single rounding.
//
// Private word layout. The make step stores each word with the code of
// k = 8r + i in nibble slot (i >> 1) + 4 * (i & 1), i.e. slots 0..7 hold
// k-offsets 0,2,4,6,1,3,5,7. Then (w >> 4j) & 0x000F000F selects the codes of
// k-offsets 2j (low half) and 2j + 1 (high half), so the four unpacked
// registers hold the eight values in natural k order, which is the order of
// the eight fp16 activations an MFMA lane loads with one 16-byte read.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace q4dev {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

__host__ __device__ constexpr int slot_of(int i) { return (i >> 1) + 4 * (i & 1); }

constexpr uint32_t kMagic2 = 0x64006400u;     // (1024.0, 1024.0) in fp16

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& f)
{
    static_assert(sizeof(To) == sizeof(From), "size");
    return __builtin_bit_cast(To, f);
}

// The zero point z of a column in the two forms the unpack subtracts: 1024 + z
// and -(64 + z), each in both halves. (64 + z has binary16 exponent 6, whose
// fraction ulp is 1/16, so its bits are 0x5400 + 16 z.)
struct zero_t {
    h2 hz;            // 1024 + z
    h2 nz16;          // -(64 + z)
    uint32_t magic;   // kMagic2, the OR constant of the unpack (a register)
};

// From a group word (scale bits | z << 16, z < 256): one v_perm_b32 puts z
// (byte 2) under 0x64 (byte 1 of magic) in both halves, 1024 + z (exact for
// z < 1024), and -(64 + z) = 960 - (1024 + z) is one exact packed subtract.
// `magic` is kMagic2; a kernel that keeps it in a register across its loop
// passes that register, so that neither this nor the unpack rebuilds it.
__device__ __forceinline__ zero_t zero_pair_sz(uint32_t sz, uint32_t magic = kMagic2)
{
    zero_t r;
    r.hz = bitcast<h2>(__builtin_amdgcn_perm(magic, sz, 0x05020502u));
    r.nz16 = bitcast<h2>(0x63806380u) - r.hz;   // (960, 960)
    r.magic = magic;
    return r;
}

__device__ __forceinline__ zero_t zero_pair(uint32_t z) { return zero_pair_sz(z << 16); }

// s in both halves (s given as binary16 bits).
__device__ __forceinline__ h2 scale_pair(uint32_t s_bits)
{
    return bitcast<h2>((s_bits & 0xFFFFu) * 0x00010001u);
}

// r = (a & mask) | orv. gfx9-family VOP3 encodings take no literal operands
// and read at most one SGPR, so this is one v_and_or_b32 only when orv is
// already in a VGPR (the mask goes to an SGPR): kernels keep the OR constant
// in a register they hide from constant folding and pass it in (an inline-asm
// v_and_or_b32 would do the same, but the compiler does not see an asm
// block's register writes when it spaces them from matrix instructions still
// writing the same registers).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t orv)
{
    return (a & mask) | orv;
}

// Unpack one private-layout word and subtract the zero point: eight fp16
// values (q - z) in k order, each a small integer, exact in fp16
// (|q - z| <= 15). Pair j (k-offsets 2j, 2j + 1) sits in nibble slots j and
// j + 4, i.e. bits 4j and 16 + 4j:
//  * pairs 0 and 2 (bits 0 and 16 of w and of w >> 8) are OR-ed into the
//    fraction of 0x6400, giving 1024 + q, and (1024 + q) - (1024 + z) is
//    exact;
//  * pairs 1 and 3 are masked where they sit (bits 4 and 20), giving
//    1024 + 16 q, and one fused multiply-add (1024 + 16 q) / 16 - (64 + z) =
//    q - z is exact as well (a power-of-two scaling and a sum of small
//    integers), which saves the shifts that would line them up.
__device__ __forceinline__ h8 sub_zero_word(uint32_t w, zero_t z)
{
    const uint32_t magic = z.magic;
    const uint32_t w8 = w >> 8;
    const h2 sixteenth = bitcast<h2>(0x2C002C00u);     // (1/16, 1/16)
    const h2 v0 = bitcast<h2>(and_or(w, 0x000F000Fu, magic)) - z.hz;
    const h2 v1 = __builtin_elementwise_fma(bitcast<h2>(and_or(w, 0x00F000F0u, magic)), sixteenth, z.nz16);
    const h2 v2 = bitcast<h2>(and_or(w8, 0x000F000Fu, magic)) - z.hz;
    const h2 v3 = __builtin_elementwise_fma(bitcast<h2>(and_or(w8, 0x00F000F0u, magic)), sixteenth, z.nz16);
    return h8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// Dequantize one private-layout word into eight fp16 values in k order:
// RNE(s * (q - z)), the exact difference times the scale, rounded once.
__device__ __forceinline__ h8 dequant_word(uint32_t w, zero_t z, h2 s2)
{
    const h8 d = sub_zero_word(w, z);
    const h8 s8 = h8{s2[0], s2[1], s2[0], s2[1], s2[0], s2[1], s2[0], s2[1]};
    return d * s8;
}

// ---- 8-bit codes -------------------------------------------------------------
// A k-step's eight 8-bit codes are two words, one byte each in k order. One
// v_perm_b32 per pair puts codes k, k + 1 into the low bytes of two fp16
// halves whose high bytes are 0x64: 1024 + q exactly (q <= 255 fits the
// 10-bit fraction). (1024 + q) - (1024 + z) is exact (|q - z| <= 255), so the
// 4-bit forms carry over: the exact q - z, or its one rounding with s.
__device__ __forceinline__ uint32_t byte_pair(uint32_t w, uint32_t sel)
{
    return __builtin_amdgcn_perm(0x64646464u, w, sel);
}

constexpr uint32_t kPairLo = 0x04010400u;   // bytes 0, 1 of w under 0x64
constexpr uint32_t kPairHi = 0x04030402u;   // bytes 2, 3

__device__ __forceinline__ h8 sub_zero_word8(uint32_t w0, uint32_t w1, zero_t z)
{
    const h2 v0 = bitcast<h2>(byte_pair(w0, kPairLo)) - z.hz;
    const h2 v1 = bitcast<h2>(byte_pair(w0, kPairHi)) - z.hz;
    const h2 v2 = bitcast<h2>(byte_pair(w1, kPairLo)) - z.hz;
    const h2 v3 = bitcast<h2>(byte_pair(w1, kPairHi)) - z.hz;
    return h8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

__device__ __forceinline__ h8 dequant_word8(uint32_t w0, uint32_t w1, zero_t z, h2 s2)
{
    const h8 d = sub_zero_word8(w0, w1, z);
    const h8 s8 = h8{s2[0], s2[1], s2[0], s2[1], s2[0], s2[1], s2[0], s2[1]};
    return d * s8;
}

// ---- bfloat16 activations ---------------------------------------------------
// The activation dtype is kept (GPTQModel wiki "Inference Backends", hardware
// table, ExLlama v2 row: FP16/BF16 activations, FP16 scales, FP32
// accumulation). With bfloat16 activations the MFMA takes bfloat16 operands,
// so the weights are formed in fp32 and packed to bfloat16 (the upper half of
// a binary32 word):
//  * the unpacked halves h = 1024 + q (pairs 0, 2) and 1024 + 16 q (pairs 1,
//    3) give f * h + c = t * (q - z) exactly in one fused multiply-add each
//    (v_fma_mix_f32 reads the fp16 half directly), with f = t, c =
//    -(1024 + z) t for pairs 0 and 2, f = t / 16, c = -(64 + z) t for pairs 1
//    and 3. For t = 1 the result is the exact small integer q - z; for t = s
//    (an fp16 scale, 11 significant bits) the constants and the product
//    t (q - z) need at most 22 bits, so each step is exact in fp32;
//  * the pack rounds to nearest even: exact for q - z, the one rounding of
//    s (q - z) to bfloat16 otherwise.
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));
typedef float ff2 __attribute__((ext_vector_type(2)));

struct mix_t {
    float t;          // scale of the result (1 for q - z)
    float c0;         // -(1024 + z) t
    float c1;         // -(64 + z) t
    uint32_t magic;   // kMagic2, the OR constant of the unpack (a register)
};

__device__ __forceinline__ mix_t mix_consts(uint32_t z, float t, uint32_t magic = kMagic2)
{
    mix_t m;
    m.t = t;
    m.c0 = -(1024.0f + (float)z) * t;
    m.c1 = -(64.0f + (float)z) * t;
    m.magic = magic;
    return m;
}

// Two fp32 values rounded to bfloat16 (nearest, ties to even), packed
// (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return bitcast<uint32_t>(__builtin_convertvector(ff2{lo, hi}, b2));
}

__device__ __forceinline__ uint32_t mix_pair(uint32_t hp, float f, float c)
{
    const h2 h = bitcast<h2>(hp);
    return pack_bf16(__builtin_fmaf((float)h[0], f, c), __builtin_fmaf((float)h[1], f, c));
}

// One k-step of 8-bit codes (two words) as eight bfloat16 values t * (q - z):
// every half is 1024 + q, so each pair takes f = t, c = -(1024 + z) t
// (exact: 11-bit products and |t (q - z)| needs at most 19 bits).
__device__ __forceinline__ b8 mix_word8(uint32_t w0, uint32_t w1, const mix_t& m)
{
    u4 o;
    o[0] = mix_pair(byte_pair(w0, kPairLo), m.t, m.c0);
    o[1] = mix_pair(byte_pair(w0, kPairHi), m.t, m.c0);
    o[2] = mix_pair(byte_pair(w1, kPairLo), m.t, m.c0);
    o[3] = mix_pair(byte_pair(w1, kPairHi), m.t, m.c0);
    return bitcast<b8>(o);
}

// One private-layout word as eight bfloat16 values t * (q - z) in k order.
__device__ __forceinline__ b8 mix_word(uint32_t w, const mix_t& m)
{
    const uint32_t magic = m.magic;
    const uint32_t w8 = w >> 8;
    const float f1 = m.t * 0.0625f;
    u4 o;
    o[0] = mix_pair(and_or(w, 0x000F000Fu, magic), m.t, m.c0);
    o[1] = mix_pair(and_or(w, 0x00F000F0u, magic), f1, m.c1);
    o[2] = mix_pair(and_or(w8, 0x000F000Fu, magic), m.t, m.c0);
    o[3] = mix_pair(and_or(w8, 0x00F000F0u, magic), f1, m.c1);
    return bitcast<b8>(o);
}

// ---- raw buffer loads ------------------------------------------------------
// A raw buffer descriptor carries the byte size of the tensor; a load whose
// per-lane offset lies at or beyond it returns zeros without touching memory.
// The kernels use that for ragged edges instead of branches: an invalid lane
// or k-step gets an offset of at least kOOB (2^31; every tensor is smaller),
// or a whole wave's load goes through a descriptor of size 0.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr uint32_t kOOB = 0x80000000u;
constexpr int kBufferDword3 = 0x00020000;   // gfx9-family raw buffer: 32-bit data format

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kBufferDword3);
}

// off: per-lane byte offset; soff: a wave-uniform byte offset added to it
// (held in a scalar register, so a per-block step costs no vector ALU).
__device__ __forceinline__ u4 buf_load16(rsrc_t r, uint32_t off, uint32_t soff = 0)
{
    return bitcast<u4>(__builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, 0));
}

// The same with the non-temporal hint (cache policy nt): for data read
// exactly once, such as the skinny kernel's weights, which then do not
// displace lines that are reused.
__device__ __forceinline__ u4 buf_load16_nt(rsrc_t r, uint32_t off, uint32_t soff = 0)
{
    constexpr int kNonTemporal = 2;
    return bitcast<u4>(__builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, kNonTemporal));
}

__device__ __forceinline__ u2 buf_load8(rsrc_t r, uint32_t off, uint32_t soff = 0)
{
    return bitcast<u2>(__builtin_amdgcn_raw_buffer_load_b64(r, (int)off, (int)soff, 0));
}

__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off, uint32_t soff = 0)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, (int)soff, 0);
}

// A 4-byte load with the non-temporal hint.
__device__ __forceinline__ uint32_t buf_load4_nt(rsrc_t r, uint32_t off, uint32_t soff = 0)
{
    constexpr int kNonTemporal = 2;
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, (int)soff, kNonTemporal);
}

__device__ __forceinline__ uint32_t buf_load2(rsrc_t r, uint32_t off, uint32_t soff = 0)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, (int)soff, 0);
}

// A 2-byte store; like the loads, a store at or past the descriptor's size
// is dropped.
__device__ __forceinline__ void buf_store2(rsrc_t r, uint32_t off, uint32_t soff, uint16_t v)
{
    __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, (int)soff, 0);
}

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x mfma32(h8 a, h8 b, f16x c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f4 mfma16(b8 a, b8 b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x mfma32(b8 a, b8 b, f16x c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v)
{
    return bitcast<uint16_t>(static_cast<_Float16>(v));
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b)
{
    return static_cast<float>(bitcast<_Float16>(b));
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v)
{
    return bitcast<uint16_t>(static_cast<__bf16>(v));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b)
{
    return bitcast<float>((uint32_t)b << 16);
}

// Activation-format traits: BF selects bfloat16 activations, bias and output.
template <bool BF>
__device__ __forceinline__ float act_to_f32(uint16_t b)
{
    if constexpr (BF) return bf16_bits_to_f32(b);
    else return f16_bits_to_f32(b);
}

template <bool BF>
__device__ __forceinline__ uint16_t f32_to_act(float v)
{
    if constexpr (BF) return f32_to_bf16_bits(v);
    else return f32_to_f16_bits(v);
}

}  // namespace q4dev
