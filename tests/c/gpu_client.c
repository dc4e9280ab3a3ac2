/* A plain C client that runs the in-place ring on the GPU through include/rr.h,
   with no Python in between: R virtual ranks of int32 (exact arithmetic) in
   separate device allocations, a SUM AllReduce with predecessor hand-offs and a
   MAX AllReduce with a counting barrier per hop, each checked on the host
   against the definition (every rank ends with the elementwise sum / maximum of
   all inputs), plus the plan query's algorithmic byte count 5 (R-1) N. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rr.h"

#define RANKS 8
#define COUNT (RANKS * 4 * 1000 + 13) /* ragged: the last chunk is short */

static int failures = 0;

#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);       \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static uint32_t next_random(uint32_t *state) { /* a 32-bit LCG: inputs only */
    *state = *state * 1664525u + 1013904223u;
    return *state >> 8;
}

static void load(void *const *bufs, const int32_t *host) {
    for (int r = 0; r < RANKS; ++r)
        EXPECT(hipMemcpy(bufs[r], host + (size_t)r * COUNT, COUNT * sizeof(int32_t),
                         hipMemcpyHostToDevice) == hipSuccess);
}

static void compare(void *const *bufs, const int32_t *want, int32_t *out, const char *what) {
    for (int r = 0; r < RANKS; ++r) {
        EXPECT(hipMemcpy(out, bufs[r], COUNT * sizeof(int32_t), hipMemcpyDeviceToHost) ==
               hipSuccess);
        for (int i = 0; i < COUNT; ++i) {
            if (out[i] != want[i]) {
                fprintf(stderr, "FAILED %s: rank %d element %d: %d, expected %d\n", what, r, i,
                        out[i], want[i]);
                ++failures;
                return;
            }
        }
    }
}

int main(void) {
    int32_t *host = malloc((size_t)RANKS * COUNT * sizeof(int32_t));
    int32_t *sum = malloc(COUNT * sizeof(int32_t));
    int32_t *max = malloc(COUNT * sizeof(int32_t));
    int32_t *out = malloc(COUNT * sizeof(int32_t));
    void *bufs[RANKS];
    hipStream_t stream;
    rr_error_record_t rec;
    rr_options_t opt;
    rr_plan_t plan;
    uint32_t state = 2024u;
    if (!host || !sum || !max || !out) return 2;

    for (int r = 0; r < RANKS; ++r)
        for (int i = 0; i < COUNT; ++i)
            host[(size_t)r * COUNT + i] = (int32_t)(next_random(&state) % 2001u) - 1000;
    for (int i = 0; i < COUNT; ++i) {
        sum[i] = 0;
        max[i] = host[i];
        for (int r = 0; r < RANKS; ++r) {
            const int32_t v = host[(size_t)r * COUNT + i];
            sum[i] += v;
            if (v > max[i]) max[i] = v;
        }
    }
    EXPECT(hipStreamCreate(&stream) == hipSuccess);
    for (int r = 0; r < RANKS; ++r)
        EXPECT(hipMalloc(&bufs[r], COUNT * sizeof(int32_t)) == hipSuccess);

    load(bufs, host);
    EXPECT(allreduce_ring(bufs, RANKS, COUNT, RR_INT32, RR_SUM, 4, stream) == RR_OK);
    EXPECT(hipStreamSynchronize(stream) == hipSuccess);
    EXPECT(rr_last_kernel_error(stream, &rec) == RR_OK);
    compare(bufs, sum, out, "SUM, predecessor hand-offs");

    load(bufs, host);
    memset(&opt, 0, sizeof opt);
    opt.sync = RR_SYNC_BARRIER;
    EXPECT(allreduce_ring_ex(bufs, RANKS, COUNT, RR_INT32, RR_MAX, 3, &opt, stream) == RR_OK);
    EXPECT(hipStreamSynchronize(stream) == hipSuccess);
    EXPECT(rr_last_kernel_error(stream, &rec) == RR_OK);
    compare(bufs, max, out, "MAX, counting barrier");

    EXPECT(rr_plan_query(RANKS, COUNT, RR_INT32, 4, 0, NULL, &plan) == RR_OK);
    EXPECT(plan.hbm_bytes == 5ull * (RANKS - 1) * COUNT * sizeof(int32_t));
    EXPECT(plan.sync == RR_SYNC_P2P && plan.launches == 1);

    for (int r = 0; r < RANKS; ++r) EXPECT(hipFree(bufs[r]) == hipSuccess);
    EXPECT(hipStreamDestroy(stream) == hipSuccess);
    rr_finalize();
    free(host);
    free(sum);
    free(max);
    free(out);
    printf("%s\n", failures ? "FAILED" : "ok");
    return failures != 0;
}
