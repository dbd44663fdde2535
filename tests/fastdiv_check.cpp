// Host check of the GEMM's launch-time divider (gptq_bit_weight_amd/csrc/
// q4_fastdiv.h) against the hardware division: every divisor up to 70000
// with random and boundary numerators, two million random (n, d) pairs over
// the whole 31-bit range with the multiples of d and their neighbours, and
// every power of two. Prints "ok" and exits 0 when all agree.
#include "q4_fastdiv.h"

#include <cstdio>
#include <random>

int main()
{
    std::mt19937_64 g(20261203);
    long long bad = 0, checked = 0;
    auto check = [&](long long n, uint32_t d, q4::FastDiv f) {
        if (n < 0 || n >= (1LL << 31)) return;
        ++checked;
        if (q4::fast_div((uint32_t)n, f) != (uint32_t)n / d && bad++ < 5)
            std::printf("n=%lld d=%u: %u, expected %u\n", n, d, q4::fast_div((uint32_t)n, f), (uint32_t)n / d);
    };
    for (uint32_t d = 1; d <= 70000; ++d) {
        const q4::FastDiv f = q4::make_fastdiv(d);
        for (int k = 0; k < 32; ++k) check((long long)(g() & 0x7FFFFFFFu), d, f);
        for (long long q = 0; q < 4; ++q)
            for (int e = -1; e <= 1; ++e) check(q * d + e, d, f);
        const long long top = ((1LL << 31) - 1) / d * d;
        for (int e = -1; e <= 1; ++e) check(top + e, d, f);
    }
    for (int t = 0; t < 2000000; ++t) {
        const uint32_t d = 1 + (uint32_t)(g() % 0x7FFFFFFFu);
        const q4::FastDiv f = q4::make_fastdiv(d);
        const long long n = (long long)(g() & 0x7FFFFFFFu);
        check(n, d, f);
        const long long m = n / d * d;
        for (int e = -1; e <= 1; ++e) check(m + e, d, f);
    }
    for (int l = 0; l < 31; ++l) {
        const uint32_t d = 1u << l;
        const q4::FastDiv f = q4::make_fastdiv(d);
        for (long long n : {0LL, 1LL, (long long)d - 1, (long long)d, (long long)d + 1, (1LL << 31) - 1}) check(n, d, f);
    }
    if (bad) {
        std::printf("%lld of %lld quotients wrong\n", bad, checked);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
