/* A plain C program that uses libar.so on the GPU with no Python and no
 * torch: device buffers from hipMalloc, inputs and results through
 * hipMemcpy, every entry point family called through include/ar.h.
 * Integer-valued inputs make every result a closed form (exact sums in any
 * order), so the program needs no reference implementation.  Prints one
 * line per check and exits non-zero on the first mismatch. */
#define _POSIX_C_SOURCE 200112L   /* setenv */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ar.h"

#define N 6
#define COUNT 10007   /* ragged: chunks of 1667 and 1668 elements */

static int fail_hip(hipError_t e, const char* what) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 1;
}

static int check_ar(ar_result_t rc, const char* what) {
    if (rc != AR_SUCCESS) {
        fprintf(stderr, "%s: %s (%s)\n", what, ar_get_error_string(rc), ar_get_last_error_detail());
        return 1;
    }
    return 0;
}

int main(void) {
    float* host = (float*)malloc(sizeof(float) * COUNT * N);
    float* back = (float*)malloc(sizeof(float) * COUNT);
    void* send[N];
    void* recv[N];
    hipStream_t stream;
    hipError_t e;
    if (host == NULL || back == NULL) return 1;
    /* the staged form with one tile of results per segment: 6 segments, 12 launches */
    if (setenv("AR_STAGE_BYTES", "8192", 1) != 0) return 1;
    if ((e = hipStreamCreate(&stream)) != hipSuccess) return fail_hip(e, "hipStreamCreate");
    for (int r = 0; r < N; ++r) {
        if ((e = hipMalloc(&send[r], sizeof(float) * COUNT)) != hipSuccess) return fail_hip(e, "hipMalloc");
        if ((e = hipMalloc(&recv[r], sizeof(float) * COUNT)) != hipSuccess) return fail_hip(e, "hipMalloc");
        for (int i = 0; i < COUNT; ++i) host[r * COUNT + i] = (float)((i * 7 + r * 3) % 17 - 8);
        e = hipMemcpy(send[r], host + (size_t)r * COUNT, sizeof(float) * COUNT, hipMemcpyHostToDevice);
        if (e != hipSuccess) return fail_hip(e, "hipMemcpy");
    }

    const ar_algo_t algos[] = {AR_ALGO_FUSED, AR_ALGO_RING, AR_ALGO_PHASES, AR_ALGO_TREE, AR_ALGO_TREE_STEPS,
                               AR_ALGO_RING_PERSISTENT, AR_ALGO_RING_PIPELINED, AR_ALGO_STAGED};
    const char* names[] = {"fused", "ring", "phases", "tree", "tree_steps", "ring_persistent", "ring_pipelined",
                           "staged"};
    for (size_t k = 0; k < sizeof(algos) / sizeof(algos[0]); ++k) {
        if (check_ar(ar_allreduce_ex((const void* const*)send, recv, COUNT, AR_FLOAT32, AR_SUM, N, algos[k], NULL, 0,
                                     stream), names[k]))
            return 1;
        if ((e = hipStreamSynchronize(stream)) != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
        for (int r = 0; r < N; ++r) {
            e = hipMemcpy(back, recv[r], sizeof(float) * COUNT, hipMemcpyDeviceToHost);
            if (e != hipSuccess) return fail_hip(e, "hipMemcpy");
            for (int i = 0; i < COUNT; ++i) {
                float want = 0.0f;
                for (int q = 0; q < N; ++q) want += host[q * COUNT + i];
                if (back[i] != want) {
                    fprintf(stderr, "%s: rank %d element %d: %g, want %g\n", names[k], r, i, back[i], want);
                    return 1;
                }
            }
        }
        printf("allreduce %s ok\n", names[k]);
    }

    /* a persistent plan, started twice, and the reduce-scatter / all-gather pair */
    ar_plan_t plan = NULL;
    if (check_ar(ar_allreduce_init((const void* const*)send, recv, COUNT, AR_FLOAT32, AR_MAX, N, AR_ALGO_FUSED, NULL,
                                   0, &plan), "init"))
        return 1;
    for (int rep = 0; rep < 2; ++rep)
        if (check_ar(ar_plan_start(plan, stream), "start")) return 1;
    ar_plan_free(plan);
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
    e = hipMemcpy(back, recv[N - 1], sizeof(float) * COUNT, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail_hip(e, "hipMemcpy");
    for (int i = 0; i < COUNT; ++i) {
        float want = host[i];
        for (int q = 1; q < N; ++q) want = host[q * COUNT + i] > want ? host[q * COUNT + i] : want;
        if (back[i] != want) {
            fprintf(stderr, "plan max: element %d: %g, want %g\n", i, back[i], want);
            return 1;
        }
    }
    printf("plan max ok\n");

    void* shard[N];
    for (int r = 0; r < N; ++r) {
        size_t b = 0, en = 0;
        if (check_ar(ar_chunk_range(r, COUNT, N, &b, &en), "chunk_range")) return 1;
        shard[r] = (char*)recv[r] + b * sizeof(float);   /* in place: shard r inside recv[r] */
    }
    if (check_ar(ar_reduce_scatter((const void* const*)send, shard, COUNT, AR_FLOAT32, AR_SUM, N, stream), "rs"))
        return 1;
    if (check_ar(ar_all_gather((const void* const*)shard, recv, COUNT, AR_FLOAT32, N, stream), "ag")) return 1;
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
    for (int r = 0; r < N; ++r) {
        e = hipMemcpy(back, recv[r], sizeof(float) * COUNT, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return fail_hip(e, "hipMemcpy");
        for (int i = 0; i < COUNT; ++i) {
            float want = 0.0f;
            for (int q = 0; q < N; ++q) want += host[q * COUNT + i];
            if (back[i] != want) {
                fprintf(stderr, "rs+ag: rank %d element %d: %g, want %g\n", r, i, back[i], want);
                return 1;
            }
        }
    }
    printf("reduce_scatter + all_gather ok\n");

    /* the pipelined ring's reduce-scatter keeps its partials in a caller-owned workspace */
    size_t ws_bytes = ar_workspace_bytes(AR_COLL_REDUCE_SCATTER, AR_ALGO_RING_PIPELINED, COUNT, AR_FLOAT32, N);
    void* ws = NULL;
    if (ws_bytes == (size_t)-1 || ws_bytes == 0) {
        fprintf(stderr, "ar_workspace_bytes: %zu\n", ws_bytes);
        return 1;
    }
    if ((e = hipMalloc(&ws, ws_bytes)) != hipSuccess) return fail_hip(e, "hipMalloc");
    for (int r = 0; r < N; ++r)
        if ((e = hipMemset(recv[r], 0, sizeof(float) * COUNT)) != hipSuccess) return fail_hip(e, "hipMemset");
    if (check_ar(ar_reduce_scatter_ex((const void* const*)send, shard, COUNT, AR_FLOAT32, AR_SUM, N,
                                      AR_ALGO_RING_PIPELINED, ws, ws_bytes, stream), "rs pipelined"))
        return 1;
    if (check_ar(ar_all_gather_ex((const void* const*)shard, recv, COUNT, AR_FLOAT32, N, AR_ALGO_RING_PIPELINED,
                                  NULL, 0, stream), "ag pipelined"))
        return 1;
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
    for (int r = 0; r < N; ++r) {
        e = hipMemcpy(back, recv[r], sizeof(float) * COUNT, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return fail_hip(e, "hipMemcpy");
        for (int i = 0; i < COUNT; ++i) {
            float want = 0.0f;
            for (int q = 0; q < N; ++q) want += host[q * COUNT + i];
            if (back[i] != want) {
                fprintf(stderr, "pipelined rs+ag: rank %d element %d: %g, want %g\n", r, i, back[i], want);
                return 1;
            }
        }
    }
    hipFree(ws);
    printf("pipelined reduce_scatter + all_gather ok\n");

    for (int r = 0; r < N; ++r) {
        hipFree(send[r]);
        hipFree(recv[r]);
    }
    hipStreamDestroy(stream);
    free(host);
    free(back);
    printf("ar.h GPU checks passed\n");
    return 0;
}
