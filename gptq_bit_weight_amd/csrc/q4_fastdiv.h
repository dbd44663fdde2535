// Division of 31-bit unsigned integers by a divisor fixed at launch time, as
// a multiply-high, an add and a shift (Granlund and Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994, section 4: the
// multiplier m' = floor(2^32 (2^l - d) / d) + 1 with l = ceil(log2 d)).
//
// The GEMM's work split needs several divisions by the number of k-tiles,
// column tiles and workgroups at the start of every workgroup; written as
// plain 64-bit or 32-bit divisions they compile to long scalar sequences.
// The host builds the divisor once per launch; a kernel divides with two
// scalar instructions.
//
// Valid for 1 <= d < 2^31 and 0 <= n < 2^31 (then n + mulhi(n, m) < 2^32 and
// the 32-bit sum cannot wrap). Header-only and free of HIP types, so the
// host compiler can check it exhaustively on the CPU.
#pragma once

#include <cstdint>

#if defined(__HIPCC__)
#define Q4_HD __host__ __device__
#else
#define Q4_HD
#endif

namespace q4 {

struct FastDiv {
    uint32_t m;   // multiplier
    uint32_t l;   // shift, ceil(log2 d)
};

inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
    return FastDiv{(uint32_t)m, l};
}

Q4_HD inline uint32_t fast_div(uint32_t n, FastDiv d)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return (n + __umulhi(n, d.m)) >> d.l;
#else
    return (uint32_t)((n + (uint32_t)(((uint64_t)n * d.m) >> 32)) >> d.l);
#endif
}

}  // namespace q4
