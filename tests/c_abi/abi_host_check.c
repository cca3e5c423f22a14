/* A plain C consumer of include/ar.h: compiled with gcc, linked against
 * libar.so, run without a GPU.  It exercises the host-side calls (chunk
 * bounds, sizes, error strings, argument validation, empty plans) and exits
 * non-zero on the first mismatch.  Fake device addresses are only compared,
 * never dereferenced: every call below returns before touching a device. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ar.h"

static int failures = 0;
#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond); \
            ++failures;                                               \
        }                                                             \
    } while (0)

int main(void) {
    size_t b = 0, e = 0;
    /* floor chunks of 1003 elements over 5 ranks: 200, 201, 200, 201, 201 */
    const size_t want[6] = {0, 200, 401, 601, 802, 1003};
    for (int c = 0; c < 5; ++c) {
        CHECK(ar_chunk_range(c, 1003, 5, &b, &e) == AR_SUCCESS);
        CHECK(b == want[c] && e == want[c + 1]);
    }
    /* 64-bit: the last chunk of 64 x (2^26 + 7) */
    CHECK(ar_chunk_range(63, ((size_t)1 << 26) + 7, 64, &b, &e) == AR_SUCCESS);
    CHECK(e == ((size_t)1 << 26) + 7 && e - b == ((size_t)1 << 20) + 1);
    CHECK(ar_chunk_range(5, 1003, 5, &b, &e) == AR_ERR_INVALID_ARGUMENT);
    CHECK(strlen(ar_get_last_error_detail()) > 0);

    CHECK(ar_dtype_size(AR_FLOAT32) == 4 && ar_dtype_size(AR_BFLOAT16) == 2 && ar_dtype_size(AR_FLOAT16) == 2);
    CHECK(strcmp(ar_get_error_string(AR_SUCCESS), "success") == 0);
    CHECK(ar_workspace_bytes(AR_COLL_REDUCE_SCATTER, AR_ALGO_RING, 1000, AR_FLOAT32, 8) == 4000 + 1024);
    CHECK(ar_workspace_bytes(AR_COLL_ALLREDUCE, AR_ALGO_FUSED, 1000, AR_FLOAT32, 8) == 0);

    const uintptr_t base = (uintptr_t)0x7f0000000000ull, S = (uintptr_t)1 << 20;
    const void* sends[4];
    void* recvs[4];
    for (int r = 0; r < 4; ++r) {
        sends[r] = (const void*)(base + r * S);
        recvs[r] = (void*)(base + (8 + r) * S);
    }
    CHECK(ar_allreduce(sends, recvs, 100, AR_FLOAT32, (ar_op_t)9, 4, NULL) == AR_ERR_INVALID_ARGUMENT);
    CHECK(ar_allreduce(sends, recvs, 100, AR_FLOAT32, AR_SUM, 0, NULL) == AR_ERR_INVALID_ARGUMENT);
    void* clash[4] = {recvs[0], recvs[0], recvs[2], recvs[3]};
    CHECK(ar_allreduce(sends, clash, 100, AR_FLOAT32, AR_SUM, 4, NULL) == AR_ERR_INVALID_ARGUMENT);
    CHECK(ar_allreduce(sends, recvs, 0, AR_FLOAT32, AR_SUM, 4, NULL) == AR_SUCCESS);

    ar_plan_t plan = NULL;
    CHECK(ar_allreduce_init(sends, recvs, 0, AR_BFLOAT16, AR_AVG, 4, AR_ALGO_RING, NULL, 0, &plan) == AR_SUCCESS);
    CHECK(plan != NULL && ar_plan_num_launches(plan) == 0);
    CHECK(ar_plan_start(plan, NULL) == AR_SUCCESS);
    CHECK(ar_plan_limit_blocks(plan, 16) == AR_SUCCESS);
    CHECK(ar_plan_limit_blocks(NULL, 16) == AR_ERR_INVALID_ARGUMENT);
    CHECK(ar_plan_free(plan) == AR_SUCCESS);

    if (failures == 0) printf("ar.h host checks passed\n");
    return failures == 0 ? 0 : 1;
}
