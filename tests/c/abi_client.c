/* A plain C99 client of include/rr.h.  It must compile as C with every warning an
   error, link against librr.so, and get the answers the header documents for
   calls that are decided on the host (argument checks, no-ops, status strings),
   so it runs without a GPU.  It also prints the size and field offsets of every
   struct the header declares, for comparison with the Python binding's layouts. */
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include "rr.h"

static int failures = 0;

#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);       \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

#define FIELD(type, f) printf(" %s=%zu", #f, offsetof(type, f))

static void layouts(void) {
    printf("rr_options_t size=%zu", sizeof(rr_options_t));
    FIELD(rr_options_t, sync); FIELD(rr_options_t, team); FIELD(rr_options_t, block);
    FIELD(rr_options_t, rounds); FIELD(rr_options_t, timeout_ns); FIELD(rr_options_t, inject);
    FIELD(rr_options_t, flags); FIELD(rr_options_t, depth); FIELD(rr_options_t, reserved);
    printf("\nrr_plan_t size=%zu", sizeof(rr_plan_t));
    FIELD(rr_plan_t, sync); FIELD(rr_plan_t, team); FIELD(rr_plan_t, block);
    FIELD(rr_plan_t, grid); FIELD(rr_plan_t, launches); FIELD(rr_plan_t, xcd_map);
    FIELD(rr_plan_t, cooperative); FIELD(rr_plan_t, resident_max); FIELD(rr_plan_t, rounds);
    FIELD(rr_plan_t, depth); FIELD(rr_plan_t, fused); FIELD(rr_plan_t, stream_loads);
    FIELD(rr_plan_t, alternate); FIELD(rr_plan_t, reserved);
    FIELD(rr_plan_t, chunk_len); FIELD(rr_plan_t, slice_len); FIELD(rr_plan_t, sub_len);
    FIELD(rr_plan_t, hbm_bytes);
    printf("\nrr_error_record_t size=%zu", sizeof(rr_error_record_t));
    FIELD(rr_error_record_t, status); FIELD(rr_error_record_t, ctx);
    FIELD(rr_error_record_t, waiter); FIELD(rr_error_record_t, hop);
    FIELD(rr_error_record_t, peer); FIELD(rr_error_record_t, reserved);
    FIELD(rr_error_record_t, expected); FIELD(rr_error_record_t, observed);
    printf("\n");
}

int main(void) {
    /* addresses that are never dereferenced: every call below is decided on the host */
    char *const base = (char *)(size_t)0x10000000u;
    void *pair[2] = {base, base + 4096};
    void *nulls[2] = {NULL, NULL};
    void *misaligned[2] = {base + 4, base + 4096};
    void *overlapping[2] = {base, base + 16}; /* 16 fp32 = 64 bytes each */
    void *one[1] = {base};
    const void *csend[2] = {base, base + 4096};
    void *crecv[2] = {base + 8192, base + 12288};
    rr_options_t opt;
    rr_counting_barrier_t *barrier = NULL;
    rr_plan_t plan;

    layouts();
    EXPECT(rr_abi_version() == RR_ABI_VERSION);
    EXPECT(strcmp(rr_status_string(RR_OK), "RR_OK") == 0);
    EXPECT(strstr(rr_status_string(RR_ERR_INVALID), "invalid") != NULL);
    EXPECT(strstr(rr_status_string(RR_ERR_TIMEOUT), "timed out") != NULL);
    EXPECT(strstr(rr_status_string((rr_status_t)77), "unknown") != NULL);

    /* the in-place ring: argument checks */
    EXPECT(allreduce_ring(NULL, 2, 16, RR_FP32, RR_SUM, 1, NULL) == RR_ERR_INVALID);
    EXPECT(allreduce_ring(pair, 0, 16, RR_FP32, RR_SUM, 1, NULL) == RR_ERR_INVALID);
    EXPECT(allreduce_ring(pair, RR_MAX_RANKS + 1, 16, RR_FP32, RR_SUM, 1, NULL) == RR_ERR_INVALID);
    EXPECT(allreduce_ring(pair, 2, 16, RR_FP32, RR_SUM, 0, NULL) == RR_ERR_INVALID);
    EXPECT(allreduce_ring(pair, 2, 16, RR_FP32, RR_SUM, RR_MAX_SLICES + 1, NULL) == RR_ERR_INVALID);
    EXPECT(allreduce_ring(pair, 2, 16, (rr_dtype_t)99, RR_SUM, 1, NULL) == RR_ERR_INVALID);
    EXPECT(allreduce_ring(pair, 2, 16, RR_FP32, (rr_op_t)99, 1, NULL) == RR_ERR_INVALID);
    EXPECT(allreduce_ring(nulls, 2, 16, RR_FP32, RR_SUM, 1, NULL) == RR_ERR_INVALID);
    EXPECT(allreduce_ring(misaligned, 2, 16, RR_FP32, RR_SUM, 1, NULL) == RR_ERR_INVALID);
    EXPECT(allreduce_ring(overlapping, 2, 16, RR_FP32, RR_SUM, 1, NULL) == RR_ERR_INVALID);
    EXPECT(reduce_scatter_ring(overlapping, 2, 16, RR_BF16, RR_MAX, 1, NULL) == RR_ERR_INVALID);
    EXPECT(all_gather_ring(misaligned, 2, 16, RR_INT32, 1, NULL) == RR_ERR_INVALID);
    /* no-ops: one rank, or no elements */
    EXPECT(allreduce_ring(one, 1, 16, RR_FP32, RR_SUM, 1, NULL) == RR_OK);
    EXPECT(allreduce_ring(pair, 2, 0, RR_FP16, RR_PROD, 3, NULL) == RR_OK);

    memset(&opt, 0, sizeof opt);
    opt.block = 192;
    EXPECT(allreduce_ring_ex(pair, 2, 16, RR_FP32, RR_SUM, 1, &opt, NULL) == RR_ERR_INVALID);
    opt.block = 0;
    opt.depth = 5;
    EXPECT(allreduce_ring_ex(pair, 2, 16, RR_FP32, RR_SUM, 1, &opt, NULL) == RR_ERR_INVALID);
    opt.depth = 0;
    opt.team = -1;
    EXPECT(reduce_scatter_ring_ex(pair, 2, 16, RR_FP32, RR_SUM, 1, &opt, NULL) == RR_ERR_INVALID);
    opt.team = 0;
    opt.sync = 99;
    EXPECT(all_gather_ring_ex(pair, 2, 16, RR_FP32, 1, &opt, NULL) == RR_ERR_INVALID);

    /* out-of-place collectives */
    EXPECT(allreduce_ring_staged(NULL, crecv, 2, 16, RR_FP32, RR_SUM, 1, NULL, NULL) ==
           RR_ERR_INVALID);
    EXPECT(alltoall(csend, (void *const *)overlapping, 2, 16, RR_FP32, NULL, NULL) ==
           RR_ERR_INVALID);
    EXPECT(alltoall(csend, crecv, 2, 0, RR_FP32, NULL, NULL) == RR_OK);

    /* barrier objects and plans */
    EXPECT(counting_barrier_create(0, 1, &barrier) == RR_ERR_INVALID);
    EXPECT(counting_barrier_create(2, 0, &barrier) == RR_ERR_INVALID);
    EXPECT(counting_barrier_create(RR_MAX_RANKS + 1, 1, &barrier) == RR_ERR_INVALID);
    EXPECT(counting_barrier_create(2, 1, NULL) == RR_ERR_INVALID);
    EXPECT(counting_barrier_destroy(NULL) == RR_OK);
    EXPECT(rr_plan_query(2, 16, RR_FP32, 1, 0, NULL, NULL) == RR_ERR_INVALID);
    EXPECT(rr_plan_query(2, 16, RR_FP32, 1, 7, NULL, &plan) == RR_ERR_INVALID);
    EXPECT(rr_plan_query(0, 16, RR_FP32, 1, 0, NULL, &plan) == RR_ERR_INVALID);

    rr_finalize();
    printf("%s\n", failures ? "FAILED" : "ok");
    return failures != 0;
}
