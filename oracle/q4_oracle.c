/*
 * q4_oracle.c -- CPU oracle for the fused GPTQ 4-bit dequantize-and-multiply.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The GPU library never links, loads or
 * calls it, and this file shares no code with it.
 *
 * What it computes (plain definition, double accumulation):
 *
 *   y[m,n] = sum_k x[m,k] * W[k,n],   W[k,n] = s[g(k),n] * (q[k,n] - z[g(k),n])
 *
 * Sources:
 *  - "GPTQ's 'Exllama Kernel Not Installed' Warning", section "Why the kernel
 *    is missing": each 32-bit word of a checkpoint carries several 4-bit
 *    codes, and every group of input rows has its own scale and zero point.
 *  - same page, section "What the fallback actually does": the fused kernel
 *    unpacks and dequantizes inside the multiply-accumulate; the fallback
 *    materializes the dequantized matrix and then runs an ordinary matmul;
 *    the two must produce identical products. Both routes are written out
 *    below.
 *  - "Implementation: Predibase Lorax GPTQ Exllama V1", I/O contract table:
 *    qweight int32, qzeros int32, scales fp16, optional g_idx int32, bits = 4,
 *    groupsize = input features per group, output fp16.
 *  - GPTQModel wiki "Inference Backends", hardware table (ExLlama v2 row):
 *    FP16 scales, FP32 accumulation. Section "Numeric epilogues": bias is
 *    added to the wide accumulator before the single final cast.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - Nibble order: code of input row k = 8r+i sits in bits 4i..4i+3 of
 *    qweight word (r, n); zero of column n = 8c+j in bits 4j..4j+3 of qzeros
 *    word (g, c). Words are read as their unsigned 32-bit pattern (nibble 7
 *    sets the sign bit of the int32).
 *  - No zero-point offset: the stored nibble is z itself.
 *  - No stored zeros (qzeros NULL): a symmetric layer, whose zero point is
 *    2^(bits-1) = 8 for every group and column (GPTQModel wiki "Inference
 *    Backends", section "Packing, conversion, and runtime initialization",
 *    packing-control row "Missing zeros": symmetric modules synthesize
 *    2 ** (bits - 1)).
 *  - g(k) = g_idx[k] when g_idx is given, else k / G. groupsize <= 0 means a
 *    single group (G = K). The number of groups is ceil(K / G).
 *  - The dequantized value in fp32, s * (q - z), is exact (an 11-bit
 *    significand times an integer of magnitude <= 15 needs <= 15 bits).
 *    Its fp16 form dq16 is one round-to-nearest-even of that exact product.
 *  - Accumulation is in double, in increasing k; the bias (if any) is added
 *    in double after the sum.
 *  - Bit width: 4 (eight codes a word) or 8 (four codes a word), packed the
 *    same way (code i of a word in bits i*bits ..; qweight along K, qzeros
 *    along N). GPTQModel wiki "Inference Backends": GPTQ kernels declare 4-
 *    and 8-bit weights (backend catalogue), and the native 8-bit GPTQ path
 *    keeps the same checkpoint tensors, qweight, qzeros, scales and g_idx
 *    (section "Runtime cache lifetime"). A symmetric 8-bit layer's zero
 *    point is 2^(8-1) = 128 (the "Missing zeros" row, as for 4-bit).
 *  - Activation format: GPTQModel wiki "Inference Backends", hardware table
 *    (ExLlama v2 row), keeps the activation dtype (FP16, BF16 or FP32) with
 *    FP16 scales and FP32 accumulation. The matmul entry points with a format
 *    argument read x and the bias as binary16 (xfmt 0) or bfloat16 (xfmt 1);
 *    the weights are the same either way. q4o_dequant_bf16 gives the weight
 *    rounded once to bfloat16, RNE_bf16(s * (q - z)).
 *
 * Error returns: 0 = OK, 1 = bad shape/argument, 2 = g_idx out of range.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------------
 * binary16 conversions, written from the IEEE 754 binary16 definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent field 0
 * holds zero and subnormals (f * 2^-24), field 31 holds inf and NaN.
 * ------------------------------------------------------------------------- */

double q4o_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* Round a non-negative double to the nearest integer, ties to even. */
static double rne_int(double r)
{
    double fl = floor(r);
    double d = r - fl;
    if (d > 0.5) return fl + 1.0;
    if (d < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* Round a double to the nearest binary16 value, ties to even.
 * For a finite |v| with binade exponent E (2^E <= |v| < 2^(E+1)), the
 * binary16 spacing is 2^(E-10) for E >= -14 and 2^-24 below. With E clamped
 * to >= -14 and n = rne(|v| / 2^(E-10)), the encoding is (E+14)*1024 + n:
 * this is continuous across binades (n = 2048 carries into the next exponent)
 * and into the subnormals (E = -14 gives the raw subnormal fraction n).
 * Any encoding >= 0x7C00 is an overflow to infinity. */
uint16_t q4o_double_to_half_rne(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return (uint16_t)(sign | 0x7E00);
    if (isinf(a)) return (uint16_t)(sign | 0x7C00);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);          /* a = m * 2^e2, m in [0.5, 1) -> E = e2 - 1 */
    int E = e2 - 1;
    if (E < -14) E = -14;
    if (E > 15) return (uint16_t)(sign | 0x7C00);
    double n = rne_int(ldexp(a, 10 - E));   /* exact scaling by a power of 2 */
    double enc = (double)(E + 14) * 1024.0 + n;
    if (enc >= 31744.0) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)enc);
}

/* ---------------------------------------------------------------------------
 * bfloat16 conversions, from its definition: the upper half of a binary32
 * word -- 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits; exponent
 * field 0 holds zero and subnormals (f * 2^-133), field 255 inf and NaN.
 * ------------------------------------------------------------------------- */

double q4o_bf16_to_double(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xFF;
    int f = b & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);
    return sign ? -v : v;
}

/* Round a double to the nearest bfloat16 value, ties to even: the binary16
 * construction above with 7 fraction bits and exponent range -126..127. The
 * spacing is 2^(E-7) for E >= -126 and 2^-133 below; the encoding
 * (E+126)*128 + n carries across binades and into the subnormals; any
 * encoding >= 0x7F80 is an overflow to infinity. */
uint16_t q4o_double_to_bf16_rne(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;
    if (E < -126) E = -126;
    if (E > 127) return (uint16_t)(sign | 0x7F80);
    double n = rne_int(ldexp(a, 7 - E));
    double enc = (double)(E + 126) * 128.0 + n;
    if (enc >= 32640.0) return (uint16_t)(sign | 0x7F80);
    return (uint16_t)(sign | (uint16_t)enc);
}

void q4o_bf16_to_double_array(int64_t n, const uint16_t* in, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = q4o_bf16_to_double(in[i]);
}

void q4o_double_to_bf16_array(int64_t n, const double* in, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = q4o_double_to_bf16_rne(in[i]);
}

typedef double (*to_double_fn)(uint16_t);

/* xfmt 0: binary16, 1: bfloat16; NULL for anything else. */
static to_double_fn format_of(int xfmt)
{
    return xfmt == 0 ? q4o_half_to_double : xfmt == 1 ? q4o_bf16_to_double : NULL;
}

void q4o_half_to_double_array(int64_t n, const uint16_t* in, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = q4o_half_to_double(in[i]);
}

void q4o_double_to_half_array(int64_t n, const double* in, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = q4o_double_to_half_rne(in[i]);
}

/* ---------------------------------------------------------------------------
 * Unpacking and group lookup. A layer has bits = 4 (eight codes a word) or
 * 8 (four codes a word), packed the same way: code i of a word sits in bits
 * i*bits .. i*bits + bits - 1, qweight along K, qzeros along N.
 * ------------------------------------------------------------------------- */

typedef struct {
    const int32_t* qweight;
    const int32_t* qzeros;     /* NULL: symmetric, zero point 2^(bits-1) */
    const uint16_t* scales;
    const int32_t* g_idx;
    int64_t N, G;
    int bits;
} layer_t;

static inline unsigned field(int32_t word, int i, int bits)
{
    return ((uint32_t)word >> (bits * i)) & ((1u << bits) - 1u);
}

/* q[k][n]: code of input row k, output column n. */
static inline unsigned code_q(const layer_t* L, int64_t k, int64_t n)
{
    const int per = 32 / L->bits;
    return field(L->qweight[(k / per) * L->N + n], (int)(k % per), L->bits);
}

/* z[g][n]: zero point of group g, column n; 2^(bits-1) for a symmetric layer
 * stored without zeros (qzeros NULL). */
static inline unsigned code_z(const layer_t* L, int64_t g, int64_t n)
{
    if (!L->qzeros) return 1u << (L->bits - 1);
    const int per = 32 / L->bits;
    return field(L->qzeros[g * (L->N / per) + n / per], (int)(n % per), L->bits);
}

static inline int64_t group_of(const layer_t* L, int64_t k)
{
    return L->g_idx ? (int64_t)L->g_idx[k] : k / L->G;
}

static int check_args(int64_t M, int64_t K, int64_t N, int64_t* G, const int32_t* g_idx, int bits)
{
    if (bits != 4 && bits != 8) return 1;
    if (M < 0 || K <= 0 || N <= 0 || K % 8 || N % 8) return 1;
    if (*G <= 0) *G = K;
    int64_t ng = (K + *G - 1) / *G;
    if (g_idx)
        for (int64_t k = 0; k < K; ++k)
            if (g_idx[k] < 0 || g_idx[k] >= ng) return 2;
    return 0;
}

static layer_t make_layer(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                          const int32_t* g_idx, int64_t N, int64_t G, int bits)
{
    layer_t L = {qweight, qzeros, scales, g_idx, N, G, bits};
    return L;
}

int q4o_num_groups(int64_t K, int64_t G)
{
    if (G <= 0) G = K;
    return (int)((K + G - 1) / G);
}

int q4o_unpack_qweight_ex(const int32_t* qweight, int64_t K, int64_t N, int bits, uint8_t* q)
{
    if ((bits != 4 && bits != 8) || K <= 0 || N <= 0 || K % (32 / bits)) return 1;
    layer_t L = make_layer(qweight, NULL, NULL, NULL, N, K, bits);
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            q[k * N + n] = (uint8_t)code_q(&L, k, n);
    return 0;
}

int q4o_unpack_qzeros_ex(const int32_t* qzeros, int64_t ng, int64_t N, int bits, uint8_t* z)
{
    if ((bits != 4 && bits != 8) || ng <= 0 || N <= 0 || N % (32 / bits)) return 1;
    layer_t L = make_layer(NULL, qzeros, NULL, NULL, N, 1, bits);
    for (int64_t g = 0; g < ng; ++g)
        for (int64_t n = 0; n < N; ++n)
            z[g * N + n] = (uint8_t)code_z(&L, g, n);
    return 0;
}

int q4o_unpack_qweight(const int32_t* qweight, int64_t K, int64_t N, uint8_t* q)
{
    return q4o_unpack_qweight_ex(qweight, K, N, 4, q);
}

int q4o_unpack_qzeros(const int32_t* qzeros, int64_t ng, int64_t N, uint8_t* z)
{
    return q4o_unpack_qzeros_ex(qzeros, ng, N, 4, z);
}

/* W[k][n] = s * (q - z) in fp32 (exact, see the header; with 8-bit codes
 * |q - z| <= 255, an 11-bit significand times an 8-bit integer). */
static inline float dequant_one(const layer_t* L, int64_t k, int64_t n)
{
    int64_t g = group_of(L, k);
    float s = (float)q4o_half_to_double(L->scales[g * L->N + n]);
    float d = (float)((int)code_q(L, k, n) - (int)code_z(L, g, n));
    return s * d;
}

/* out: 0 fp32 W, 1 binary16 RNE(W), 2 bfloat16 RNE(W). */
static int dequant_any(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                       const int32_t* g_idx, int64_t K, int64_t N, int64_t G, int bits, int out,
                       void* dst)
{
    int rc = check_args(0, K, N, &G, g_idx, bits);
    if (rc) return rc;
    layer_t L = make_layer(qweight, qzeros, scales, g_idx, N, G, bits);
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            float w = dequant_one(&L, k, n);
            if (out == 0) ((float*)dst)[k * N + n] = w;
            else if (out == 1) ((uint16_t*)dst)[k * N + n] = q4o_double_to_half_rne((double)w);
            else ((uint16_t*)dst)[k * N + n] = q4o_double_to_bf16_rne((double)w);
        }
    return 0;
}

int q4o_dequant32_ex(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                     const int32_t* g_idx, int64_t K, int64_t N, int64_t G, int bits, float* W)
{
    return dequant_any(qweight, qzeros, scales, g_idx, K, N, G, bits, 0, W);
}

/* dq16[k][n] = RNE_fp16(s * (q - z)), binary16 bit patterns. */
int q4o_dequant16_ex(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                     const int32_t* g_idx, int64_t K, int64_t N, int64_t G, int bits, uint16_t* dq)
{
    return dequant_any(qweight, qzeros, scales, g_idx, K, N, G, bits, 1, dq);
}

/* dqb[k][n] = RNE_bf16(s * (q - z)), bfloat16 bit patterns. */
int q4o_dequant_bf16_ex(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                        const int32_t* g_idx, int64_t K, int64_t N, int64_t G, int bits, uint16_t* dq)
{
    return dequant_any(qweight, qzeros, scales, g_idx, K, N, G, bits, 2, dq);
}

int q4o_dequant32(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                  const int32_t* g_idx, int64_t K, int64_t N, int64_t G, float* W)
{
    return q4o_dequant32_ex(qweight, qzeros, scales, g_idx, K, N, G, 4, W);
}

int q4o_dequant16(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                  const int32_t* g_idx, int64_t K, int64_t N, int64_t G, uint16_t* dq)
{
    return q4o_dequant16_ex(qweight, qzeros, scales, g_idx, K, N, G, 4, dq);
}

int q4o_dequant_bf16(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                     const int32_t* g_idx, int64_t K, int64_t N, int64_t G, uint16_t* dq)
{
    return q4o_dequant_bf16_ex(qweight, qzeros, scales, g_idx, K, N, G, 4, dq);
}

/* ---------------------------------------------------------------------------
 * The two routes to y. Both sum in increasing k in double and add the bias
 * last, so they are bit-identical by construction; the test suite checks it.
 * x and the bias are read in format xfmt (0 binary16, 1 bfloat16).
 * ------------------------------------------------------------------------- */

/* Fused route: dequantize each weight inside the k loop, never store W. */
int q4o_matmul_fused_ex(int xfmt, int bits, const uint16_t* x, const int32_t* qweight,
                        const int32_t* qzeros, const uint16_t* scales, const int32_t* g_idx,
                        const uint16_t* bias, int64_t M, int64_t K, int64_t N, int64_t G,
                        double* y, double* A)
{
    to_double_fn to_d = format_of(xfmt);
    if (!to_d) return 1;
    int rc = check_args(M, K, N, &G, g_idx, bits);
    if (rc) return rc;
    layer_t L = make_layer(qweight, qzeros, scales, g_idx, N, G, bits);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aabs = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double w = (double)dequant_one(&L, k, n);
                double p = to_d(x[m * K + k]) * w;
                acc += p;
                aabs += fabs(p);
            }
            if (bias) acc += to_d(bias[n]);
            y[m * N + n] = acc;
            if (A) A[m * N + n] = aabs;
        }
    return 0;
}

/* Fallback route: materialize the dequantized W[K][N], then a plain matmul. */
int q4o_matmul_fallback_ex(int xfmt, int bits, const uint16_t* x, const int32_t* qweight,
                           const int32_t* qzeros, const uint16_t* scales, const int32_t* g_idx,
                           const uint16_t* bias, int64_t M, int64_t K, int64_t N, int64_t G,
                           double* y)
{
    to_double_fn to_d = format_of(xfmt);
    if (!to_d) return 1;
    int rc = check_args(M, K, N, &G, g_idx, bits);
    if (rc) return rc;
    float* W = (float*)malloc((size_t)K * (size_t)N * sizeof(float));
    if (!W) return 1;
    q4o_dequant32_ex(qweight, qzeros, scales, g_idx, K, N, G, bits, W);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += to_d(x[m * K + k]) * (double)W[k * N + n];
            if (bias) acc += to_d(bias[n]);
            y[m * N + n] = acc;
        }
    free(W);
    return 0;
}

/* Fused route at selected output elements (m[i], n[i]), i < count. Used for
 * full-size layers where the whole product would take the CPU too long. */
int q4o_matmul_fused_at_ex(int xfmt, int bits, const uint16_t* x, const int32_t* qweight,
                           const int32_t* qzeros, const uint16_t* scales, const int32_t* g_idx,
                           const uint16_t* bias, int64_t M, int64_t K, int64_t N, int64_t G,
                           int64_t count, const int64_t* ms, const int64_t* ns,
                           double* y, double* A)
{
    to_double_fn to_d = format_of(xfmt);
    if (!to_d) return 1;
    int rc = check_args(M, K, N, &G, g_idx, bits);
    if (rc) return rc;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return 1;
    layer_t L = make_layer(qweight, qzeros, scales, g_idx, N, G, bits);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = ms[i], n = ns[i];
        double acc = 0.0, aabs = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double w = (double)dequant_one(&L, k, n);
            double p = to_d(x[m * K + k]) * w;
            acc += p;
            aabs += fabs(p);
        }
        if (bias) acc += to_d(bias[n]);
        y[i] = acc;
        if (A) A[i] = aabs;
    }
    return 0;
}

/* binary16 activations, 4-bit weights (the original entry points). */
int q4o_matmul_fused(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                     const uint16_t* scales, const int32_t* g_idx, const uint16_t* bias,
                     int64_t M, int64_t K, int64_t N, int64_t G, double* y, double* A)
{
    return q4o_matmul_fused_ex(0, 4, x, qweight, qzeros, scales, g_idx, bias, M, K, N, G, y, A);
}

int q4o_matmul_fallback(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                        const uint16_t* scales, const int32_t* g_idx, const uint16_t* bias,
                        int64_t M, int64_t K, int64_t N, int64_t G, double* y)
{
    return q4o_matmul_fallback_ex(0, 4, x, qweight, qzeros, scales, g_idx, bias, M, K, N, G, y);
}

int q4o_matmul_fused_at(const uint16_t* x, const int32_t* qweight, const int32_t* qzeros,
                        const uint16_t* scales, const int32_t* g_idx, const uint16_t* bias,
                        int64_t M, int64_t K, int64_t N, int64_t G,
                        int64_t count, const int64_t* ms, const int64_t* ns,
                        double* y, double* A)
{
    return q4o_matmul_fused_at_ex(0, 4, x, qweight, qzeros, scales, g_idx, bias, M, K, N, G,
                                  count, ms, ns, y, A);
}

int q4o_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the parallel loops use from now on (n >= 1); returns the previous
 * count. Only the timing of a CPU baseline uses it: the results do not depend
 * on it (each output element is one sequential sum over k). */
int q4o_set_num_threads(int n)
{
    int prev = q4o_num_threads();
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
    return prev;
}
