/*
 * ring_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU model of the ring AllReduce, written to
 * check the GPU library against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.  It
 * shares no code, header, table or helper with the GPU library.
 *
 * What it follows (the post "Why AllReduce = ReduceScatter + AllGather -- with
 * NCCL Ring AllReduce" on loosp.cn):
 *   - section 1: every rank ends with S_k = the reduction over all ranks of
 *     chunk k;
 *   - section 4: ranks form the ring 0 -> 1 -> ... -> R-1 -> 0; each rank
 *     receives from its predecessor and sends to its successor;
 *   - section 5: ReduceScatter takes R-1 rounds.  In round 1 rank r sends its
 *     own chunk r; in every later round it forwards the partial it received in
 *     the round before.  The receiver folds the incoming partial into its own
 *     copy of the same chunk (incoming first, e.g. "a0 + b0" at GPU1).  After
 *     the last round rank r holds the finished chunk (r + 1) mod R;
 *   - section 6: AllGather takes R-1 rounds of receive + copy + send with no
 *     arithmetic; every rank forwards what it received in the round before;
 *   - section 12: the tensor is cut into R contiguous pieces, one per rank;
 *   - sections 8-10: the same loop as the staged primitives of one rank (Table
 *     V of the paper the post discusses): step 0 send, steps 1..R-2
 *     recvReduceSend, step R-1 recvReduceCopySend, steps R..2R-3 recvCopySend,
 *     step 2R-2 recv -- data arrive in a receive buffer, are reduced with or
 *     copied from the rank's input, land in its output, and go on to the next
 *     rank's receive buffer (ro_staged_allreduce);
 *   - sections 2-3: ReduceScatter leaves every reduced chunk on one rank and
 *     AllGather copies them to all; which rank keeps which chunk depends on the
 *     numbering.  ro_reduce_scatter_nccl and ro_all_gather_nccl use the
 *     numbering of the standalone collectives (rank r keeps chunk r; rank r's
 *     input becomes block r of every output).
 *
 * Readings where the page is silent (each is listed in the design notes):
 *   - chunk boundaries: chunk_len = ceil(count / R) rounded up to a whole
 *     16-byte vector; chunk c = [c*chunk_len, min((c+1)*chunk_len, count)),
 *     possibly empty;
 *   - int32 SUM wraps modulo 2^32;
 *   - fp32 SUM is one IEEE binary32 addition per hop (round to nearest even);
 *   - bf16 SUM is one correctly rounded bfloat16 addition per hop: the exact
 *     sum rounded to nearest even at 8 significant bits (overflow to infinity,
 *     subnormals kept, any NaN becomes the quiet NaN 0x7FC0);
 *   - MAX keeps the incoming value unless the local value compares greater;
 *     MIN keeps it unless the local value compares less;
 *   - PROD: int32 wraps modulo 2^32; fp32 is one binary32 multiplication; bf16
 *     and fp16 are one correctly rounded multiplication in the storage format
 *     (the exact product rounded once, ties to even).  A binary32 product
 *     rounded to the storage format gives the same bits: for fp16 the binary32
 *     product is exact; for bf16 it has at most 16 significant bits, too few
 *     for a binary32 rounding below the normal range to create a tie at 8 bits;
 *   - fp16 SUM is one correctly rounded binary16 addition (11 significant bits,
 *     subnormals down to 2^-24, overflow to infinity, any NaN becomes 0x7E00);
 *     binary32 addition followed by rounding to fp16 gives the same bits,
 *     because 24 >= 2*11 + 2;
 *   - the staged loop keeps a receive buffer of two slots per rank: the
 *     message of step k goes to slot k mod 2, so a rank never overwrites the
 *     slot its successor is still to read.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared (no fast-math, no
 * OpenMP, no vector intrinsics).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { RO_INT32 = 0, RO_FP32 = 1, RO_BF16 = 2, RO_FP16 = 3 };
enum { RO_SUM = 0, RO_MAX = 1, RO_MIN = 2, RO_PROD = 3 };
enum { RO_OK = 0, RO_EINVAL = 1, RO_ENOMEM = 2 };
enum { RO_MAX_RANKS = 64 };

/* One hop of the ring, as recorded by the optional trace. */
typedef struct {
    int32_t phase;     /* 0 = ReduceScatter, 1 = AllGather */
    int32_t round;     /* 1 .. R-1 within the phase */
    int32_t hop;       /* 1 .. 2(R-1) over the whole AllReduce */
    int32_t src;       /* sending rank */
    int32_t dst;       /* receiving rank = (src + 1) mod R */
    int32_t chunk;     /* chunk index carried by the hop */
    uint64_t bytes;    /* bytes carried */
    int32_t nterms;    /* how many rank inputs the receiver's chunk now folds */
    uint8_t terms[RO_MAX_RANKS]; /* those ranks, in fold order */
} ro_hop_t;

typedef struct {
    ro_hop_t *hops;    /* caller-owned array */
    int32_t capacity;  /* entries available */
    int32_t used;      /* entries written */
} ro_trace_t;

static size_t elem_size(int dt) { return dt == RO_BF16 || dt == RO_FP16 ? 2u : 4u; }

static int valid_dtype(int dt)
{
    return dt == RO_INT32 || dt == RO_FP32 || dt == RO_BF16 || dt == RO_FP16;
}

static int valid_op(int op) { return op == RO_SUM || op == RO_MAX || op == RO_MIN || op == RO_PROD; }

static int mod(int a, int m) { int r = a % m; return r < 0 ? r + m : r; }

/* ---------------------------------------------------------------- partition */

int ro_chunk_bounds(uint64_t count, int R, int dt, uint64_t *begin /* R + 1 */)
{
    if (R < 1 || R > RO_MAX_RANKS || !valid_dtype(dt) || !begin) return RO_EINVAL;
    uint64_t per_vector = 16u / elem_size(dt);
    uint64_t share = (count + (uint64_t)R - 1u) / (uint64_t)R;
    uint64_t chunk_len = (share + per_vector - 1u) / per_vector * per_vector;
    for (int c = 0; c <= R; ++c) {
        uint64_t b = (uint64_t)c * chunk_len;
        begin[c] = b < count ? b : count;
    }
    return RO_OK;
}

/* ------------------------------------------------------------- element math */

static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Nearest bfloat16 to x, ties to even.  bfloat16 keeps 8 significant bits,
 * normal exponents -126..127 and subnormals down to 2^-133.  Rounding the
 * exact sum of two bfloat16 values first to double (53 bits) and then to 8
 * bits gives the same result as rounding it once, because 53 >= 2*8 + 2. */
static uint16_t bf16_from_double(double x)
{
    if (isnan(x)) return 0x7FC0u;
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);          /* a lies in [2^(e-1), 2^e) */
    int q = e - 8;               /* weight of the last kept bit */
    if (q < -133) q = -133;      /* subnormal spacing */
    double n = nearbyint(ldexp(a, -q)); /* default mode: ties to even */
    double r = ldexp(n, q);
    if (r >= 0x1p128) return (uint16_t)(sign | 0x7F80u);
    float f = (float)r;          /* exact: at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

static double fp16_to_double(uint16_t h)
{
    int e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);
    return (h & 0x8000u) ? -v : v;
}

/* Nearest binary16 to x, ties to even: 11 significant bits, normal exponents
 * -14..15, subnormals down to 2^-24, largest finite value 65504. */
static uint16_t fp16_from_double(double x)
{
    if (isnan(x)) return 0x7E00u;
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);          /* a lies in [2^(e-1), 2^e) */
    int q = e - 11;              /* weight of the last kept bit */
    if (q < -24) q = -24;        /* subnormal spacing */
    double r = ldexp(nearbyint(ldexp(a, -q)), q);
    if (r == 0.0) return sign;   /* below half the smallest subnormal */
    if (r > 65504.0) return (uint16_t)(sign | 0x7C00u);
    int er;
    (void)frexp(r, &er);         /* r lies in [2^(er-1), 2^er) */
    if (er - 1 < -14) return (uint16_t)(sign | (uint16_t)ldexp(r, 24));
    uint16_t mant = (uint16_t)(ldexp(r, 11 - er) - 1024.0);
    return (uint16_t)(sign | (uint16_t)((er - 1 + 15) << 10) | mant);
}

/* local[i] = incoming[i] (op) local[i] for n elements. */
static void fold_range(int dt, int op, const void *incoming, void *local, uint64_t n)
{
    if (dt == RO_INT32) {
        const int32_t *in = (const int32_t *)incoming;
        int32_t *lo = (int32_t *)local;
        for (uint64_t i = 0; i < n; ++i) {
            if (op == RO_SUM)
                lo[i] = (int32_t)((uint32_t)in[i] + (uint32_t)lo[i]);
            else if (op == RO_MAX)
                lo[i] = lo[i] > in[i] ? lo[i] : in[i];
            else if (op == RO_MIN)
                lo[i] = lo[i] < in[i] ? lo[i] : in[i];
            else
                lo[i] = (int32_t)((uint32_t)in[i] * (uint32_t)lo[i]);
        }
    } else if (dt == RO_FP32) {
        const float *in = (const float *)incoming;
        float *lo = (float *)local;
        for (uint64_t i = 0; i < n; ++i) {
            if (op == RO_SUM)
                lo[i] = in[i] + lo[i];
            else if (op == RO_MAX)
                lo[i] = lo[i] > in[i] ? lo[i] : in[i];
            else if (op == RO_MIN)
                lo[i] = lo[i] < in[i] ? lo[i] : in[i];
            else
                lo[i] = in[i] * lo[i];
        }
    } else if (dt == RO_FP16) {
        const uint16_t *in = (const uint16_t *)incoming;
        uint16_t *lo = (uint16_t *)local;
        for (uint64_t i = 0; i < n; ++i) {
            double a = fp16_to_double(in[i]);
            double b = fp16_to_double(lo[i]);
            if (op == RO_SUM)
                lo[i] = fp16_from_double(a + b);
            else if (op == RO_MAX)
                lo[i] = b > a ? lo[i] : in[i];
            else if (op == RO_MIN)
                lo[i] = b < a ? lo[i] : in[i];
            else
                lo[i] = fp16_from_double(a * b);
        }
    } else {
        const uint16_t *in = (const uint16_t *)incoming;
        uint16_t *lo = (uint16_t *)local;
        for (uint64_t i = 0; i < n; ++i) {
            double a = bf16_to_float(in[i]);
            double b = bf16_to_float(lo[i]);
            if (op == RO_SUM)
                lo[i] = bf16_from_double(a + b);
            else if (op == RO_MAX)
                lo[i] = b > a ? lo[i] : in[i];
            else if (op == RO_MIN)
                lo[i] = b < a ? lo[i] : in[i];
            else
                lo[i] = bf16_from_double(a * b);  /* exact in double */
        }
    }
}

/* ------------------------------------------------------------------- trace */

/* Fold order of every (rank, chunk) slot, kept only when a trace is asked for. */
typedef struct {
    int R;
    uint8_t *terms;  /* [R][R][R]: ranks folded into slot (rank, chunk) */
    int32_t *nterms; /* [R][R] */
} provenance_t;

static int provenance_init(provenance_t *p, int R)
{
    p->R = R;
    p->terms = (uint8_t *)calloc((size_t)R * R * R, 1);
    p->nterms = (int32_t *)calloc((size_t)R * R, sizeof(int32_t));
    if (!p->terms || !p->nterms) return RO_ENOMEM;
    for (int r = 0; r < R; ++r)
        for (int c = 0; c < R; ++c) {
            p->nterms[r * R + c] = 1;
            p->terms[((size_t)r * R + c) * R] = (uint8_t)r;
        }
    return RO_OK;
}

static void provenance_free(provenance_t *p)
{
    free(p->terms);
    free(p->nterms);
}

static void record_hop(ro_trace_t *tr, provenance_t *pv, int phase, int round, int hop,
                       int src, int dst, int chunk, uint64_t bytes)
{
    int R = pv->R;
    uint8_t *from = pv->terms + ((size_t)src * R + chunk) * R;
    uint8_t *to = pv->terms + ((size_t)dst * R + chunk) * R;
    int nfrom = pv->nterms[src * R + chunk];
    int nto = pv->nterms[dst * R + chunk];
    if (phase == 0) {
        /* receiver's chunk becomes incoming terms followed by its own terms */
        uint8_t merged[RO_MAX_RANKS];
        int n = 0;
        for (int i = 0; i < nfrom && n < RO_MAX_RANKS; ++i) merged[n++] = from[i];
        for (int i = 0; i < nto && n < RO_MAX_RANKS; ++i) merged[n++] = to[i];
        memcpy(to, merged, (size_t)n);
        pv->nterms[dst * R + chunk] = n;
    } else {
        memcpy(to, from, (size_t)nfrom);
        pv->nterms[dst * R + chunk] = nfrom;
    }
    if (tr->used < tr->capacity) {
        ro_hop_t *h = &tr->hops[tr->used];
        memset(h, 0, sizeof *h);
        h->phase = phase;
        h->round = round;
        h->hop = hop;
        h->src = src;
        h->dst = dst;
        h->chunk = chunk;
        h->bytes = bytes;
        h->nterms = pv->nterms[dst * R + chunk];
        memcpy(h->terms, to, (size_t)h->nterms);
    }
    tr->used++;
}

/* --------------------------------------------------------------- the ring */

static int check_args(void *const *bufs, int R, int dt, int op)
{
    if (R < 1 || R > RO_MAX_RANKS || !valid_dtype(dt)) return RO_EINVAL;
    if (!valid_op(op)) return RO_EINVAL;
    if (!bufs) return RO_EINVAL;
    for (int r = 0; r < R; ++r)
        if (!bufs[r]) return RO_EINVAL;
    return RO_OK;
}

/* ReduceScatter rounds.  In round s rank r passes chunk (r - s + 1) mod R to
 * rank (r + 1) mod R, which folds it into its own copy.  The R transfers of one
 * round touch disjoint slots, so doing them one after another in rank order is
 * the same as doing them at once. */
static void reduce_scatter_rounds(void *const *bufs, int R, const uint64_t *begin, int dt,
                                  int op, ro_trace_t *tr, provenance_t *pv)
{
    size_t es = elem_size(dt);
    for (int s = 1; s <= R - 1; ++s) {
        for (int r = 0; r < R; ++r) {
            int c = mod(r - s + 1, R);
            int q = (r + 1) % R;
            uint64_t lo = begin[c], n = begin[c + 1] - begin[c];
            fold_range(dt, op, (const char *)bufs[r] + lo * es, (char *)bufs[q] + lo * es, n);
            if (tr) record_hop(tr, pv, 0, s, s, r, q, c, n * es);
        }
    }
}

/* AllGather rounds.  In round t rank r forwards chunk (r + 2 - t) mod R to rank
 * (r + 1) mod R: in round 1 the chunk it finished in ReduceScatter, later the
 * chunk it received in the round before.  A plain byte copy. */
static void all_gather_rounds(void *const *bufs, int R, const uint64_t *begin, int dt,
                              int hop_offset, ro_trace_t *tr, provenance_t *pv)
{
    size_t es = elem_size(dt);
    for (int t = 1; t <= R - 1; ++t) {
        for (int r = 0; r < R; ++r) {
            int c = mod(r + 2 - t, R);
            int q = (r + 1) % R;
            uint64_t lo = begin[c], n = begin[c + 1] - begin[c];
            memcpy((char *)bufs[q] + lo * es, (const char *)bufs[r] + lo * es, n * es);
            if (tr) record_hop(tr, pv, 1, t, hop_offset + t, r, q, c, n * es);
        }
    }
}

enum { PHASE_RS = 1, PHASE_AG = 2 };

static int run_ring(void *const *bufs, int R, uint64_t count, int dt, int op, int phases,
                    ro_trace_t *trace)
{
    int rc = check_args(bufs, R, dt, op);
    if (rc != RO_OK) return rc;
    if (trace) trace->used = 0;
    if (R == 1) return RO_OK;
    uint64_t begin[RO_MAX_RANKS + 1];
    ro_chunk_bounds(count, R, dt, begin);
    provenance_t pv = {0, NULL, NULL};
    if (trace) {
        rc = provenance_init(&pv, R);
        if (rc != RO_OK) {
            provenance_free(&pv);
            return rc;
        }
    }
    if (phases & PHASE_RS) reduce_scatter_rounds(bufs, R, begin, dt, op, trace, &pv);
    if (phases & PHASE_AG)
        all_gather_rounds(bufs, R, begin, dt, (phases & PHASE_RS) ? R - 1 : 0, trace, &pv);
    if (trace) provenance_free(&pv);
    return RO_OK;
}

/* In place: bufs[r] holds rank r's `count` elements; afterwards every rank
 * holds the reduction of all ranks. */
int ro_allreduce(void *const *bufs, int R, uint64_t count, int dt, int op, ro_trace_t *trace)
{
    return run_ring(bufs, R, count, dt, op, PHASE_RS | PHASE_AG, trace);
}

/* In place: afterwards chunk (r + 1) mod R of bufs[r] is finished; chunk c of
 * bufs[r] holds the fold of ranks c, c+1, ..., r (its own input when c == r). */
int ro_reduce_scatter(void *const *bufs, int R, uint64_t count, int dt, int op,
                      ro_trace_t *trace)
{
    return run_ring(bufs, R, count, dt, op, PHASE_RS, trace);
}

/* In place: chunk (r + 1) mod R of bufs[r] is spread to every rank. */
int ro_all_gather(void *const *bufs, int R, uint64_t count, int dt, ro_trace_t *trace)
{
    return run_ring(bufs, R, count, dt, RO_SUM, PHASE_AG, trace);
}

/* The AllReduce result at single element positions.  vals[k*R + r] is rank r's
 * input at position k, which lies in chunk chunks[k]; out[k*R + r] receives rank
 * r's result.  Each position runs through ro_allreduce itself, placed in a tiny
 * problem where it falls in the same chunk, so the fold order is the ring's. */
int ro_allreduce_at(const void *vals, const int32_t *chunks, uint64_t npos, int R, int dt,
                    int op, void *out)
{
    if (R < 1 || R > RO_MAX_RANKS || !valid_dtype(dt) || !vals || !chunks || !out)
        return RO_EINVAL;
    size_t es = elem_size(dt);
    uint64_t per_vector = 16u / es;
    uint64_t count = (uint64_t)R * per_vector;
    char *store = (char *)calloc((size_t)R * count, es);
    if (!store) return RO_ENOMEM;
    void *bufs[RO_MAX_RANKS];
    for (int r = 0; r < R; ++r) bufs[r] = store + (size_t)r * count * es;
    int rc = RO_OK;
    for (uint64_t k = 0; k < npos && rc == RO_OK; ++k) {
        int c = chunks[k];
        if (c < 0 || c >= R) {
            rc = RO_EINVAL;
            break;
        }
        uint64_t at = (uint64_t)c * per_vector;
        for (int r = 0; r < R; ++r)
            memcpy((char *)bufs[r] + at * es, (const char *)vals + (k * R + r) * es, es);
        rc = ro_allreduce(bufs, R, count, dt, op, NULL);
        for (int r = 0; r < R; ++r)
            memcpy((char *)out + (k * R + r) * es, (const char *)bufs[r] + at * es, es);
    }
    free(store);
    return rc;
}

/* Order-free reference for floating-point tolerance checks: the fp64 sum of the
 * ranks' inputs and the fp64 sum of their magnitudes, per element. */
int ro_direct_sum_f64(const void *const *bufs, int R, uint64_t count, int dt, double *sum,
                      double *abs_sum)
{
    if (R < 1 || R > RO_MAX_RANKS || (dt != RO_FP32 && dt != RO_BF16 && dt != RO_FP16) || !bufs ||
        !sum)
        return RO_EINVAL;
    for (uint64_t i = 0; i < count; ++i) {
        double s = 0.0, a = 0.0;
        for (int r = 0; r < R; ++r) {
            double x = dt == RO_FP32   ? (double)((const float *)bufs[r])[i]
                       : dt == RO_BF16 ? (double)bf16_to_float(((const uint16_t *)bufs[r])[i])
                                       : fp16_to_double(((const uint16_t *)bufs[r])[i]);
            s += x;
            a += fabs(x);
        }
        sum[i] = s;
        if (abs_sum) abs_sum[i] = a;
    }
    return RO_OK;
}

/* ------------------------------------------------------- the staged loop */

/* Primitives of one step (ring post section 8). */
enum {
    PRIM_SEND = 0,               /* input -> next rank's receive buffer */
    PRIM_RECV_REDUCE_SEND = 1,   /* received (op) input -> next rank */
    PRIM_RECV_REDUCE_COPY_SEND = 2, /* received (op) input -> output and next rank */
    PRIM_RECV_COPY_SEND = 3,     /* received -> output and next rank */
    PRIM_RECV = 4,               /* received -> output */
    PRIM_RECV_REDUCE_COPY = 5,   /* received (op) input -> output (last ReduceScatter step) */
    PRIM_COPY_SEND = 6           /* input -> output and next rank (first AllGather step) */
};

/* One step of one rank, as recorded by the optional step log. */
typedef struct {
    int32_t step;
    int32_t rank;
    int32_t prim;
    int32_t chunk;
    uint64_t bytes_read;     /* from the input, the receive buffer */
    uint64_t bytes_written;  /* to the output, the next rank's receive buffer */
} ro_step_t;

typedef struct {
    ro_step_t *steps;  /* caller-owned array */
    int32_t capacity;
    int32_t used;
} ro_steplog_t;

enum { STAGED_ALLREDUCE = 0, STAGED_RS = 1, STAGED_AG = 2 };

/* The staged loop over R ranks.  mode STAGED_ALLREDUCE: send[r] and recv[r]
 * hold n elements, cut into chunks as the in-place ring does; steps 0..2R-2.
 * STAGED_RS: send[r] holds R blocks of n elements, recv[r] one block, which
 * ends as the reduction of block r; steps 0..R-1, the last one
 * recvReduceCopy.  STAGED_AG: send[r] holds n elements, recv[r] R blocks;
 * steps 0..R-1, the first one copySend.  At step k rank r handles chunk
 * (r - k) mod R (ReduceScatter: (r - k - 1) mod R, so that rank r finishes
 * chunk r).  recv may equal send for STAGED_ALLREDUCE: a rank reads each chunk
 * of its input before it writes that chunk of its output. */
static int staged(const void *const *send, void *const *recv, int R, uint64_t n, int dt, int op,
                  int mode, ro_steplog_t *log)
{
    if (R < 1 || R > RO_MAX_RANKS || !valid_dtype(dt) || !valid_op(op) || !send || !recv)
        return RO_EINVAL;
    for (int r = 0; r < R; ++r)
        if (!send[r] || !recv[r]) return RO_EINVAL;
    if (log) log->used = 0;
    size_t es = elem_size(dt);
    uint64_t begin[RO_MAX_RANKS + 1];
    if (mode == STAGED_ALLREDUCE) {
        ro_chunk_bounds(n, R, dt, begin);
    } else {
        for (int c = 0; c <= R; ++c) begin[c] = (uint64_t)c * n;
    }
    uint64_t max_len = 0;
    for (int c = 0; c < R; ++c)
        if (begin[c + 1] - begin[c] > max_len) max_len = begin[c + 1] - begin[c];
    if (R == 1) {
        /* nothing to exchange: the output is the input (block 0) */
        if ((const void *)recv[0] != send[0]) memmove(recv[0], send[0], n * es);
        return RO_OK;
    }
    /* receive buffers: two slots of one chunk per rank, plus one chunk of scratch */
    char *fifo = (char *)calloc((size_t)(2 * R + 1) * (max_len ? max_len : 1), es);
    if (!fifo) return RO_ENOMEM;
    char *val = fifo + (size_t)2 * R * max_len * es;
    int last = mode == STAGED_ALLREDUCE ? 2 * R - 2 : R - 1;
    for (int k = 0; k <= last; ++k) {
        for (int r = 0; r < R; ++r) {
            int c = mod(r - k - (mode == STAGED_RS ? 1 : 0), R);
            int has_in = k >= 1;
            int has_local, reduce, has_out, has_send, prim;
            if (mode == STAGED_ALLREDUCE) {
                has_local = k <= R - 1;
                reduce = k >= 1 && k <= R - 1;
                has_out = k >= R - 1;
                has_send = k <= 2 * R - 3;
                prim = k == 0           ? PRIM_SEND
                       : k < R - 1      ? PRIM_RECV_REDUCE_SEND
                       : k == R - 1     ? PRIM_RECV_REDUCE_COPY_SEND
                       : k < 2 * R - 2  ? PRIM_RECV_COPY_SEND
                                        : PRIM_RECV;
            } else if (mode == STAGED_RS) {
                has_local = 1;
                reduce = k >= 1;
                has_out = k == R - 1;
                has_send = k <= R - 2;
                prim = k == 0 ? PRIM_SEND : k < R - 1 ? PRIM_RECV_REDUCE_SEND : PRIM_RECV_REDUCE_COPY;
            } else {
                has_local = k == 0;
                reduce = 0;
                has_out = 1;
                has_send = k <= R - 2;
                prim = k == 0 ? PRIM_COPY_SEND : k < R - 1 ? PRIM_RECV_COPY_SEND : PRIM_RECV;
            }
            uint64_t len = begin[c + 1] - begin[c];
            const char *in = fifo + ((size_t)r * 2 + (size_t)((k + 1) & 1)) * max_len * es;
            char *next = fifo + ((size_t)((r + 1) % R) * 2 + (size_t)(k & 1)) * max_len * es;
            const char *local = (const char *)send[r] +
                                (mode == STAGED_AG ? 0 : begin[c]) * es;
            char *out = (char *)recv[r] + (mode == STAGED_RS ? 0 : begin[c]) * es;
            if (has_local) memcpy(val, local, len * es);
            if (has_in) {
                if (reduce)
                    fold_range(dt, op, in, val, len);
                else
                    memcpy(val, in, len * es);
            }
            if (has_out) memcpy(out, val, len * es);
            if (has_send) memcpy(next, val, len * es);
            if (log && log->used < log->capacity) {
                ro_step_t *st = &log->steps[log->used];
                st->step = k;
                st->rank = r;
                st->prim = prim;
                st->chunk = c;
                st->bytes_read = (uint64_t)(has_local + has_in) * len * es;
                st->bytes_written = (uint64_t)(has_out + has_send) * len * es;
            }
            if (log) log->used++;
        }
    }
    free(fifo);
    return RO_OK;
}

/* Out of place (recv may equal send): recv[r] ends with the AllReduce of the
 * ranks' send buffers, computed by the staged primitives. */
int ro_staged_allreduce(const void *const *send, void *const *recv, int R, uint64_t count,
                        int dt, int op, ro_steplog_t *log)
{
    return staged(send, recv, R, count, dt, op, STAGED_ALLREDUCE, log);
}

/* send[r]: R blocks of recvcount elements; recv[r] ends with block r reduced
 * over all ranks. */
int ro_reduce_scatter_nccl(const void *const *send, void *const *recv, int R, uint64_t recvcount,
                           int dt, int op, ro_steplog_t *log)
{
    return staged(send, recv, R, recvcount, dt, op, STAGED_RS, log);
}

/* send[r]: sendcount elements; recv[r] ends with R blocks, block q = send[q]. */
int ro_all_gather_nccl(const void *const *send, void *const *recv, int R, uint64_t sendcount,
                       int dt, ro_steplog_t *log)
{
    return staged(send, recv, R, sendcount, dt, RO_SUM, STAGED_AG, log);
}

/* ------------------------------------------------------------- AlltoAll */

/* The pure AlltoAll of the 2kiu.com article on NCCL GIN (section "a pure GIN
 * AlltoAll kernel"): every rank puts block q of its send buffer into rank q's
 * receive buffer at block position (its own rank), so recv[q] block r =
 * send[r] block q.  A byte copy; blocks of `count` elements of `es` bytes. */
int ro_alltoall(const void *const *send, void *const *recv, int R, uint64_t count, int es)
{
    if (R < 1 || R > RO_MAX_RANKS || (es != 2 && es != 4) || !send || !recv) return RO_EINVAL;
    uint64_t bytes = count * (uint64_t)es;
    for (int r = 0; r < R; ++r)
        for (int q = 0; q < R; ++q)
            memcpy((char *)recv[q] + (uint64_t)r * bytes, (const char *)send[r] + (uint64_t)q * bytes,
                   bytes);
    return RO_OK;
}

int ro_abi_version(void) { return 1; }
