/*
 * exhaustive_hop.c -- TEST HELPER: every ordered pair of 16-bit operands
 * through the CPU oracle's one-hop fold, against a reference written here.
 *
 * Usage: exhaustive_hop ORACLE_SO DTYPE DECODE_TABLE THREADS [STEP [OP]]
 *   ORACLE_SO     path of the oracle's shared library (loaded with dlopen; only
 *                 its ro_allreduce entry point is called)
 *   DTYPE         2 = bfloat16, 3 = binary16 (the oracle's dtype codes)
 *   DECODE_TABLE  65536 little-endian binary64 values: the value of every
 *                 16-bit pattern, decoded by the caller (NaN for NaN patterns)
 *   THREADS       worker threads
 *   STEP          check the first operands 0, STEP, 2*STEP, ... only (default 1:
 *                 all 65536 of them, i.e. all 2^32 ordered pairs)
 *   OP            0 = SUM (default), 1 = MAX, 2 = MIN, 3 = PROD (the oracle's codes)
 *
 * The per-hop fold of a 16-bit SUM is the exact sum of the two operands rounded
 * once to the format, nearest even (the post "Why AllReduce = ReduceScatter +
 * AllGather -- with NCCL Ring AllReduce", section 5, folds the incoming
 * partial into the local one; the rounding is the reading of the format's
 * arithmetic).  The reference here adds the two decoded values in binary64 and
 * rounds that sum to the format by integer operations on its bits.  Rounding
 * the exact sum first to binary64 and then to p significant bits equals one
 * rounding because 53 >= 2p + 2 (p = 8 or 11).  Any NaN result is the format's
 * canonical quiet NaN (0x7FC0, 0x7E00).  PROD: the product of the two decoded
 * values, exact in binary64 (at most 2p <= 22 significant bits), rounded once
 * the same way.  MAX and MIN select, with no arithmetic: the local operand if it
 * compares greater (less) than the incoming one, else the incoming one, so ties,
 * signed zeros and NaNs resolve by that rule, bit for bit.
 *
 * For each first operand a (one oracle call per a), rank 0 holds a in all 65536
 * positions and rank 1 holds every pattern b once; with R = 2 each position is
 * folded exactly once (incoming a into local b in the first chunk, positions
 * below 32768; incoming b into local a in the second), and both ranks end with
 * the folded value.
 *
 * Prints "pairs N mismatches M" and, on a mismatch, the first one.
 */
#include <dlfcn.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef int (*allreduce_fn)(void *const *, int, uint64_t, int, int, void *);

static allreduce_fn g_allreduce;
static int g_dtype;
static double g_value[65536];

/* Format parameters: significant bits p, exponent field width. */
static int g_p, g_ebits;
static uint16_t g_qnan;

/* Round a binary64 value to the 16-bit format, nearest even. */
static uint16_t round_to_format(double s)
{
    if (s != s) return g_qnan;
    uint64_t u;
    memcpy(&u, &s, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 63) << 15);
    u &= 0x7FFFFFFFFFFFFFFFull;
    const int bias = (1 << (g_ebits - 1)) - 1;
    const int emin = 1 - bias, emax = bias;
    const uint16_t inf = (uint16_t)(((1u << g_ebits) - 1u) << (g_p - 1));
    if (u == 0) return sign;
    if (u >= 0x7FF0000000000000ull) return (uint16_t)(sign | inf);
    const int biased = (int)(u >> 52);
    if (biased == 0) {
        /* a binary64 subnormal: far below half the format's smallest value */
        return sign;
    }
    int de = biased - 1023;                                  /* s in [2^de, 2^(de+1)) */
    const uint64_t m = (u & 0x000FFFFFFFFFFFFFull) | (1ull << 52); /* s = m * 2^(de-52) */
    const int ulp = (de >= emin ? de : emin) - (g_p - 1);    /* weight of the last kept bit */
    const int shift = ulp - (de - 52);                       /* low bits of m to drop */
    uint64_t q;
    if (shift >= 64) {
        q = 0; /* below a quarter of the last kept bit */
    } else {
        q = m >> shift;
        const uint64_t rem = m & ((1ull << shift) - 1ull);
        const uint64_t half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (q & 1ull))) ++q;
    }
    if (de < emin) {
        /* subnormal: the pattern is q itself; q == 2^(p-1) is the smallest normal */
        return (uint16_t)(sign | (uint16_t)q);
    }
    if (q == (1ull << g_p)) {  /* carried into the next binade */
        q >>= 1;
        ++de;
    }
    if (de > emax) return (uint16_t)(sign | inf);
    return (uint16_t)(sign | (uint16_t)((de + bias) << (g_p - 1)) |
                      (uint16_t)(q - (1ull << (g_p - 1))));
}

static int g_step = 1;
static int g_op = 0;

/* The folded pattern at position b of the call for first operand a. */
static uint16_t reference(int a, int b)
{
    if (g_op == 0) return round_to_format(g_value[a] + g_value[b]);
    if (g_op == 3) return round_to_format(g_value[a] * g_value[b]);
    const int in = b < 32768 ? a : b, lo = b < 32768 ? b : a;
    const double vin = g_value[in], vlo = g_value[lo];
    const int local_wins = g_op == 1 ? vlo > vin : vlo < vin;
    return (uint16_t)(local_wins ? lo : in);
}

typedef struct {
    int first, last; /* first operands [first, last), taken every g_step */
    uint64_t pairs, mismatches;
    int bad_a, bad_b;
    uint16_t bad_got, bad_want;
    int rc;
} job_t;

static void *worker(void *arg)
{
    job_t *j = (job_t *)arg;
    uint16_t *r0 = (uint16_t *)malloc(65536 * 2), *r1 = (uint16_t *)malloc(65536 * 2);
    if (!r0 || !r1) {
        j->rc = 2;
        free(r0);
        free(r1);
        return NULL;
    }
    void *bufs[2] = {r0, r1};
    for (int a = j->first; a < j->last; ++a) {
        if (a % g_step) continue;
        for (int b = 0; b < 65536; ++b) {
            r0[b] = (uint16_t)a;
            r1[b] = (uint16_t)b;
        }
        if (g_allreduce(bufs, 2, 65536, g_dtype, g_op, NULL) != 0) {
            j->rc = 3;
            break;
        }
        for (int b = 0; b < 65536; ++b) {
            const uint16_t want = reference(a, b);
            ++j->pairs;
            if (r0[b] != want || r1[b] != want) {
                if (j->mismatches++ == 0) {
                    j->bad_a = a;
                    j->bad_b = b;
                    j->bad_got = r0[b] != want ? r0[b] : r1[b];
                    j->bad_want = want;
                }
            }
        }
    }
    free(r0);
    free(r1);
    return NULL;
}

int main(int argc, char **argv)
{
    if (argc < 5 || argc > 7) {
        fprintf(stderr, "usage: %s ORACLE_SO DTYPE DECODE_TABLE THREADS [STEP [OP]]\n", argv[0]);
        return 2;
    }
    void *lib = dlopen(argv[1], RTLD_NOW | RTLD_LOCAL);
    if (!lib) {
        fprintf(stderr, "dlopen: %s\n", dlerror());
        return 2;
    }
    g_allreduce = (allreduce_fn)dlsym(lib, "ro_allreduce");
    if (!g_allreduce) {
        fprintf(stderr, "ro_allreduce not found\n");
        return 2;
    }
    g_dtype = atoi(argv[2]);
    if (g_dtype == 2) {
        g_p = 8;
        g_ebits = 8;
        g_qnan = 0x7FC0u;
    } else if (g_dtype == 3) {
        g_p = 11;
        g_ebits = 5;
        g_qnan = 0x7E00u;
    } else {
        fprintf(stderr, "dtype must be 2 (bf16) or 3 (fp16)\n");
        return 2;
    }
    FILE *f = fopen(argv[3], "rb");
    if (!f || fread(g_value, sizeof(double), 65536, f) != 65536) {
        fprintf(stderr, "cannot read the decode table\n");
        return 2;
    }
    fclose(f);
    if (argc >= 6) g_step = atoi(argv[5]);
    if (g_step < 1) g_step = 1;
    if (argc == 7) g_op = atoi(argv[6]);
    if (g_op < 0 || g_op > 3) {
        fprintf(stderr, "op must be 0 (SUM), 1 (MAX), 2 (MIN) or 3 (PROD)\n");
        return 2;
    }
    int nthreads = atoi(argv[4]);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    pthread_t tid[64];
    job_t jobs[64];
    memset(jobs, 0, sizeof jobs);
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].first = (int)((int64_t)65536 * t / nthreads);
        jobs[t].last = (int)((int64_t)65536 * (t + 1) / nthreads);
        if (pthread_create(&tid[t], NULL, worker, &jobs[t]) != 0) {
            fprintf(stderr, "pthread_create failed\n");
            return 2;
        }
    }
    uint64_t pairs = 0, mismatches = 0;
    int rc = 0;
    const job_t *first_bad = NULL;
    for (int t = 0; t < nthreads; ++t) {
        pthread_join(tid[t], NULL);
        pairs += jobs[t].pairs;
        mismatches += jobs[t].mismatches;
        if (jobs[t].rc) rc = jobs[t].rc;
        if (jobs[t].mismatches && !first_bad) first_bad = &jobs[t];
    }
    printf("pairs %llu mismatches %llu\n", (unsigned long long)pairs,
           (unsigned long long)mismatches);
    if (first_bad)
        printf("first a=%#06x b=%#06x got=%#06x want=%#06x\n", first_bad->bad_a, first_bad->bad_b,
               first_bad->bad_got, first_bad->bad_want);
    return rc;
}
