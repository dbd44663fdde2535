/*
 * A plain C99 client of the library: it includes q4.h as C, takes the address
 * of every call the header declares (so linking fails if one is missing or
 * not exported with C linkage), and runs the host-only calls, which need no
 * GPU. Built and run by tests/test_abi_client.py. Exit status 0 on success;
 * otherwise the number of the first failed check.
 */
#include <stdio.h>
#include <string.h>

#include "q4.h"

#define CHECK(n, cond)                                                     \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "check %d failed: %s (%s)\n", n, #cond,        \
                    q4_last_error() ? q4_last_error() : "");               \
            return n;                                                      \
        }                                                                  \
    } while (0)

/* every declared call, with the header's own types */
static struct {
    q4_matrix* (*make)(const int32_t*, const int32_t*, const uint16_t*, const int32_t*, int, int, int);
    q4_matrix* (*make_bits)(const int32_t*, const int32_t*, const uint16_t*, const int32_t*, int, int, int, int);
    q4_matrix* (*make_cat)(int, const int32_t* const*, const int32_t* const*, const uint16_t* const*,
                           const int32_t*, int, const int*, int);
    q4_matrix* (*make_cat_bits)(int, const int32_t* const*, const int32_t* const*, const uint16_t* const*,
                                const int32_t*, int, const int*, int, int);
    q4_status (*matmul)(const q4_matrix*, const uint16_t*, uint16_t*, int, hipStream_t);
    q4_status (*matmul_bias)(const q4_matrix*, const uint16_t*, const uint16_t*, uint16_t*, int, hipStream_t);
    q4_status (*matmul_ex)(const q4_matrix*, const uint16_t*, const uint16_t*, uint16_t*, int, int, int, int,
                           hipStream_t);
    q4_status (*matmul_static)(const q4_matrix*, const uint16_t*, const uint16_t*, uint16_t*, int, hipStream_t);
    q4_status (*matmul_bf16)(const q4_matrix*, const uint16_t*, const uint16_t*, uint16_t*, int, hipStream_t);
    q4_status (*matmul_ex_bf16)(const q4_matrix*, const uint16_t*, const uint16_t*, uint16_t*, int, int, int,
                                int, hipStream_t);
    void (*free_)(q4_matrix*);
    q4_status (*last_status)(void);
    const char* (*last_error)(void);
    int (*path_for)(const q4_matrix*, int);
    q4_status (*dump)(const q4_matrix*, int, uint16_t*, hipStream_t);
    q4_status (*dump_bf16)(const q4_matrix*, int, uint16_t*, hipStream_t);
    int (*gemv_gather)(const q4_matrix*, int, int);
    int (*handle_info)(const q4_matrix*, int*, int*, int*, int*);
    int (*handle_bits)(const q4_matrix*);
    q4_status (*read_probe)(const void*, size_t, uint32_t*, hipStream_t);
    q4_status (*check_shape)(int, int, int);
    q4_status (*check_shape_bits)(int, int, int, int);
    q4_status (*plan_actorder)(const int32_t*, int, int, int32_t*, int*);
    int (*plan_gemm)(int, int, int, int);
    int (*plan_gemm_waves)(int, int, int, int);
    q4_status (*plan_gemv)(int, int, int, int, int, int*, int*);
    int (*plan_gemv_gather)(int, int, int);
} api = {
    q4_make, q4_make_bits, q4_make_cat, q4_make_cat_bits, q4_matmul, q4_matmul_bias, q4_matmul_ex,
    q4_matmul_static, q4_matmul_bf16, q4_matmul_ex_bf16, q4_free, q4_last_status, q4_last_error,
    q4_path_for, q4_dequant_dump, q4_dequant_dump_bf16, q4_gemv_gather, q4_handle_info, q4_handle_bits,
    q4_read_probe, q4_check_shape, q4_check_shape_bits, q4_plan_actorder, q4_plan_gemm, q4_plan_gemm_waves, q4_plan_gemv,
    q4_plan_gemv_gather,
};

int main(void)
{
    /* argument checks */
    CHECK(1, api.check_shape(512, 512, 128) == Q4_OK);
    CHECK(2, api.check_shape(512, 510, 128) == Q4_ERR_INVALID_ARG);
    CHECK(3, api.last_status() == Q4_ERR_INVALID_ARG && strlen(api.last_error()) > 0);
    CHECK(4, api.check_shape_bits(512, 512, 128, 3) == Q4_ERR_UNSUPPORTED);

    /* act-order plan: one stable argsort of g_idx */
    {
        const int32_t g_idx[8] = {1, 0, 1, 0, 0, 1, 1, 0};
        const int32_t want[8] = {1, 3, 4, 7, 0, 2, 5, 6};
        int32_t perm[8];
        int trivial = -1;
        CHECK(5, api.plan_actorder(g_idx, 8, 4, perm, &trivial) == Q4_OK && trivial == 0);
        CHECK(6, memcmp(perm, want, sizeof want) == 0);
        const int32_t id[8] = {0, 0, 0, 0, 1, 1, 1, 1};
        CHECK(7, api.plan_actorder(id, 8, 4, perm, &trivial) == Q4_OK && trivial == 1);
    }

    /* launch plans */
    {
        int ct = 0, sp = 0;
        CHECK(8, api.plan_gemv(1, 4096, 4096, 128, 256, &ct, &sp) == Q4_OK && ct >= 1 && sp >= 1);
        CHECK(9, api.plan_gemv(Q4_GEMV_MAX_M + 1, 4096, 4096, 128, 256, &ct, &sp) == Q4_ERR_INVALID_ARG);
        CHECK(10, api.plan_gemm(2048, 11008, 4096, 256) >= 1);
        CHECK(11, api.plan_gemm(2048, 11008, 4096, 256) <= Q4_GEMM_MAX_WORKERS);
        CHECK(80, api.plan_gemm_waves(2048, 11008, 4096, 256) == 8);
        CHECK(81, api.plan_gemm_waves(64, 11008, 4096, 256) == 4);
    }

    /* calls on a null handle fail cleanly, without a GPU */
    CHECK(12, api.path_for(NULL, 1) == -1);
    CHECK(13, api.matmul(NULL, NULL, NULL, 1, NULL) == Q4_ERR_INVALID_ARG);
    api.free_(NULL);

    printf("ok\n");
    return 0;
}
