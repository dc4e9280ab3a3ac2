/*
 * rr.h -- ring AllReduce over virtual ranks on one AMD Instinct MI355X (gfx950).
 *
 * C ABI of librr.so.  Plain pointers and sizes only.
 *
 * THE OPERATION.  The post "Why AllReduce = ReduceScatter + AllGather -- with
 * NCCL Ring AllReduce" (loosp.cn) defines it:
 *   section 1  -- R ranks each hold a buffer cut into R chunks; afterwards every
 *                 rank holds S_k, the reduction over all ranks of chunk k, for
 *                 every k;
 *   section 4  -- the ranks form the ring 0 -> 1 -> ... -> R-1 -> 0;
 *   section 5  -- ReduceScatter: R-1 rounds; in round s rank r sends chunk
 *                 (r - s + 1) mod R to rank r + 1, which folds it into its own
 *                 copy (incoming first); afterwards rank r owns chunk (r+1) mod R;
 *   section 6  -- AllGather: R-1 rounds of receive + copy + send, no arithmetic;
 *                 in round t rank r forwards chunk (r + 2 - t) mod R;
 *   section 12 -- the data are cut into R contiguous pieces.
 * Here the R ranks are virtual: rank r is the device buffer bufs[r], and a
 * "send" from rank r is a store into bufs[(r + 1) mod R].  Every hop therefore
 * moves exactly the chunk traffic of the real ring: a ReduceScatter hop reads
 * the incoming chunk and the local chunk and writes the folded chunk; an
 * AllGather hop reads and writes one chunk.
 *
 * CHUNKS.  chunk_len = ceil(count / R) rounded up to a whole 16-byte vector
 * (4 int32/fp32 or 8 bf16 elements); chunk c covers elements
 * [c*chunk_len, min((c+1)*chunk_len, count)) and may be empty.  Each chunk is
 * further cut into `nslices` slices of equal nominal length (vector aligned);
 * slices only schedule work: results do not depend on nslices.
 *
 * ARITHMETIC, one fold per ReduceScatter hop, local = incoming (op) local:
 *   int32 SUM / PROD  wrap modulo 2^32
 *   fp32  SUM / PROD  one binary32 operation, round to nearest even
 *   bf16, fp16 SUM / PROD  the exact result rounded once to the format, nearest
 *              even (computed in binary32 and rounded: the same bits); a NaN
 *              result is 0x7FC0 (bf16) or 0x7E00 (fp16)
 *   MAX / MIN  the local value if it compares greater / less, else the
 *              incoming value, keeping the winner's bits (signed for int32)
 * So the element result of chunk c is the left fold over ranks c, c+1, ...,
 * c+R-1 (mod R), rounded to the storage type after every step.
 *
 * HAND-OFF.  One persistent kernel runs every hop.  Each slice is split among a
 * team of workgroups; a (slice, team member) pair is a lane, and workgroups own
 * (virtual rank, lane) pairs.  Every lane is an independent context with one
 * 64-bit signal per rank, so lanes pipeline against each other.  After a hop a
 * producer adds 1 to its consumer's signal (the counting barrier of the DeepEP
 * pull request "make the rail barrier a counting barrier", section "Fix"); the
 * consumer advances a private shadow by the number of arrivals it expects and
 * waits until the signal reaches the shadow, with the rolling comparison the
 * NCCL GIN documentation describes (2kiu.com article on NCCL GIN, section
 * "Signals and counters"), so counters never need a reset.  A signal never has
 * two producers of the same rank: an anonymous count could then be met by one
 * producer running a hop ahead while another still writes (the same pull
 * request, section "Scoped to the rail team").
 *
 * STREAMS AND ORDER.  Every entry point that takes a stream enqueues work on it
 * and returns once the work is enqueued (the status covers validation and
 * enqueue only).  Device-side failures (a wait that timed out) surface through
 * rr_last_kernel_error after the stream has drained.  Calls on one device share
 * one signal workspace, so they must not overlap in time: issue them on one
 * stream, or order them yourself.
 *
 * OWNERSHIP.  The caller owns every buffer and stream; the library never keeps
 * a buffer pointer beyond the call.  The library owns one small per-device
 * workspace (signals, shadows, the error record), allocated on the first call
 * on a device (or by rr_init) and freed by rr_finalize.  The first call on a
 * device must therefore not happen under stream capture.
 *
 * GRAPHS.  After that first call, calls may be captured into a HIP graph and
 * replayed: a call records kernel launches only (no memset or copy nodes), and
 * everything a kernel must tell apart from one launch to the next (signal
 * counts, shadows, the per-launch tag of its XCD placement check) lives in the
 * device workspace and advances on the device, so a replay behaves as a fresh
 * call.  The staged loop's receive buffers must already be large enough (a
 * call of the same or larger size made outside capture), since growing them
 * allocates.  Growing them later does not free the smaller buffers (they are
 * kept until rr_finalize), so a graph captured before a growth still replays.
 */
#ifndef RR_H
#define RR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RR_ABI_VERSION 1
#define RR_MAX_RANKS 64      /* virtual ranks per call */
#define RR_MAX_SLICES 1024   /* slices per call; slices * team * R <= 65536 */

typedef enum { RR_INT32 = 0, RR_FP32 = 1, RR_BF16 = 2, RR_FP16 = 3 } rr_dtype_t;

typedef enum { RR_SUM = 0, RR_MAX = 1, RR_MIN = 2, RR_PROD = 3 } rr_op_t;

typedef enum {
    RR_OK = 0,
    RR_ERR_INVALID = 1,     /* bad argument; nothing was enqueued */
    RR_ERR_UNSUPPORTED = 2, /* valid, but the requested mode cannot run it */
    RR_ERR_HIP = 3,         /* a HIP runtime call failed */
    RR_ERR_TIMEOUT = 4,     /* a device wait gave up (see rr_error_record_t) */
    RR_ERR_NOMEM = 5        /* device or host allocation failed */
} rr_status_t;

/* How consecutive hops hand off. */
typedef enum {
    RR_SYNC_AUTO = 0,    /* P2P when every workgroup can be resident, else LAUNCH */
    RR_SYNC_P2P = 1,     /* persistent kernel; a consumer waits for its predecessor
                            rank's workgroup in the same lane only (1 arrival per hop) */
    RR_SYNC_BARRIER = 2, /* persistent kernel; every hop ends with a counting barrier
                            over all R ranks of the lane: each workgroup adds 1 to
                            the lane's one shared signal and waits until it has
                            advanced by R (the R-1 other ranks and itself); with
                            RR_FLAG_WAITER_SIGNAL each workgroup adds 1 to every
                            other rank's own signal, a waiter expects R-1 */
    RR_SYNC_LAUNCH = 3,  /* one kernel launch per hop; stream order is the barrier */
    RR_SYNC_PER_PEER = 4 /* counting_barrier_run only: one slot per (waiter, peer);
                            each peer adds 1 to its own slot and a waiter waits for
                            every slot (the layout the DeepEP pull request replaced,
                            section "Fix"); the ring calls reject it */
} rr_sync_t;

/* Fault injection, for failure tests only.  Each makes one waiter's wait
   unsatisfiable, so that it times out and every workgroup still exits. */
#define RR_INJECT_EXTRA_EXPECTED 0x1u /* rank 0, context 0 expects one arrival too many
                                         at its first wait */
#define RR_INJECT_DROP_ARRIVAL   0x2u /* rank 0, context 0 skips its first arrival */
#define RR_INJECT_DEFER_ARRIVAL  0x4u /* counting_barrier_run, barrier modes: waiter 0 of
                                         context 0 holds back its step-1 and step-2
                                         arrivals at waiter 1 until it has passed
                                         step 2, which needs waiter 1 past step 1.
                                         A per-peer barrier (and R = 2) therefore
                                         times out naming the peer, while a counting
                                         barrier with R >= 3 passes on a stand-in
                                         from another peer one step ahead (DeepEP
                                         pull request, section "Scoped to the rail
                                         team") and completes */

/* Flags. */
#define RR_FLAG_NO_XCD_MAP       0x1u /* plain block -> (rank, lane) order; hand-offs then
                                         cross XCDs and write L2 back every hop */
#define RR_FLAG_NO_POINTER_CHECK 0x2u /* skip the per-call allocation-extent check */
#define RR_FLAG_FUSED_BOUNDARY   0x8u /* AllReduce only: the last ReduceScatter hop also
                                         stores the finished chunk in the owner's
                                         successor (the ring post's recvReduceCopySend,
                                         sections 8-9), so the first AllGather hop moves
                                         no data: 5(R-1)N - N bytes instead of 5(R-1)N */
#define RR_FLAG_AUDIT            0x10u /* counting_barrier_run, RR_SYNC_BARRIER: every
                                         arrival also bumps the sender's per-peer slot
                                         (a witness, released before the counting add);
                                         after each step a waiter counts it as an early
                                         pass if some peer's witness has not advanced.
                                         A lower bound (a witness may land just before
                                         its counting add); slower, for tests only */
#define RR_FLAG_STREAM_LOADS     0x20u /* in-place ring: mark the loads of the
                                         predecessor's buffer non-temporal (always,
                                         not only when the buffers exceed the
                                         Infinity Cache; see rr_plan_t.stream_loads) */
#define RR_FLAG_CACHED_LOADS     0x40u /* in-place ring: never mark them (both flags
                                         together: RR_ERR_INVALID) */
#define RR_FLAG_SHARED_SIGNAL    0x80u /* counting_barrier_run, RR_SYNC_BARRIER: one
                                         signal per context that every waiter adds 1 to
                                         and polls (pass expected_per_step = R); the in-
                                         place ring's barrier does this by default */
#define RR_FLAG_WAITER_SIGNAL    0x800u /* in-place ring, RR_SYNC_BARRIER: one signal per
                                         (lane, rank) instead of one per lane; after each
                                         hop a workgroup adds 1 to the R-1 other ranks'
                                         signals (R-1 atomics instead of 1) and waits for
                                         R-1 on its own.  Same results.  Not together with
                                         RR_FLAG_SHARED_SIGNAL */
#define RR_FLAG_POLL_FAST        0x100u /* in-place ring: sleep about 64 clocks between
                                          polls of a hand-off signal (the default with
                                          predecessor hand-offs, and with a barrier whose
                                          hop moves less than 64 MiB over all ranks) */
#define RR_FLAG_POLL_MEDIUM      0x200u /* ... about 512 clocks */
#define RR_FLAG_POLL_SLOW        0x400u /* ... about 4096 clocks (the default with a barrier
                                          whose hop moves 64 MiB or more).  At most one of
                                          the three poll flags (else RR_ERR_INVALID) */
#define RR_FLAG_ASCENDING        0x1000u /* in-place ring: every hop runs through its
                                          piece in ascending order (see
                                          rr_plan_t.alternate).  Same results */
#define RR_FLAG_ALTERNATE        0x2000u /* in-place ring: the even hops run from the top
                                          down, whatever the size (both flags
                                          together: RR_ERR_INVALID; the other calls
                                          ignore both) */
#define RR_FLAG_COOPERATIVE      0x4u /* launch the persistent kernel with
                                         hipLaunchCooperativeKernel (co-residency
                                         guaranteed by the runtime; otherwise the
                                         library checks grid <= resident capacity and
                                         the bounded waits catch a starved grid) */

typedef struct {
    int32_t sync;        /* rr_sync_t */
    int32_t team;        /* workgroups per (rank, slice); 0 = choose */
    int32_t block;       /* threads per workgroup: 128, 256, 512 or 1024; 0 = automatic,
                            from the lane piece p (the bytes a workgroup moves per
                            lane and hop): 128 if p <= 2 KiB, 256 if 16 KiB < p <=
                            32 KiB, 128 if p <= 64 KiB with R >= 16 and the R
                            buffers together above 256 MiB, else 512 (columns are
                            planned for 512 either way); except RR_SYNC_BARRIER
                            with R >= 16, 8 R dividing the CU count and 3 x the
                            per-rank bytes >= 1.5 GiB: 1024, columns planned for
                            one workgroup per CU */
    int32_t rounds;      /* lane groups each workgroup runs one after another
                            (depth * rounds must divide slices * team);
                            0 = choose from the buffer size */
    uint64_t timeout_ns; /* bound on every device wait; 0 = 2 s */
    uint32_t inject;     /* RR_INJECT_* */
    uint32_t flags;      /* RR_FLAG_* */
    int32_t depth;       /* lanes each workgroup interleaves hop by hop, 1..4; 0 = choose */
    int32_t reserved;    /* 0 */
} rr_options_t;

/* What a call will run (rr_plan_query). */
typedef struct {
    int32_t sync;        /* rr_sync_t actually used (never AUTO) */
    int32_t team;
    int32_t block;
    int32_t grid;        /* workgroups per launch */
    int32_t launches;    /* kernel launches per call */
    int32_t xcd_map;     /* 1 if each column of R workgroups is placed on one XCD
                            (the grid is then padded to a multiple of 8 columns) */
    int32_t cooperative; /* 1 if launched with hipLaunchCooperativeKernel */
    int32_t resident_max;/* workgroups the device can hold at once for this kernel */
    int32_t rounds;      /* lane groups each workgroup runs one after another */
    int32_t depth;       /* lanes each workgroup interleaves */
    int32_t fused;       /* 1 if the boundary hop is fused (RR_FLAG_FUSED_BOUNDARY) */
    int32_t stream_loads;/* in-place ring: 1 if the loads of the predecessor's buffer
                            are non-temporal.  By default when the R buffers together
                            exceed the 256 MB Infinity Cache: a chunk read from the
                            predecessor is not read again before it is overwritten,
                            so the hint leaves the cache to the partials each rank
                            writes for its successor; when everything fits, it only
                            evicts lines that would have hit. */
    int32_t alternate;   /* in-place ring: 1 if the even hops run through their piece
                            from the top down (the odd ones bottom up), so that a hop
                            first reads what its predecessor wrote last, which is the
                            most likely to be still in the Infinity Cache.  By default
                            when the R buffers together exceed half the cache
                            (128 MiB); below that everything stays cached either way.
                            Other calls: always 0 */
    int32_t reserved;    /* 0 */
    uint64_t chunk_len;  /* elements */
    uint64_t slice_len;  /* elements */
    uint64_t sub_len;    /* elements per team member */
    uint64_t hbm_bytes;  /* algorithmic bytes read + written by one call */
} rr_plan_t;

/* Device-side failure record (rr_last_kernel_error).  Following the DeepEP
   pull request (section "Cost": with one counting slot the stalled peer cannot
   be identified, so the timeout diagnostic gives the number of missing arrivals
   and the signal), the record gives the waiter's signal (context and rank) and
   expected - observed missing arrivals; only a per-peer barrier
   (RR_SYNC_PER_PEER) can name the peer. */
typedef struct {
    int32_t status;    /* RR_OK or RR_ERR_TIMEOUT */
    int32_t ctx;       /* context (lane = slice * team + member) of the waiter */
    int32_t waiter;    /* its virtual rank */
    int32_t hop;       /* hop (or barrier step) it was about to start */
    int32_t peer;      /* the peer that did not arrive (per-peer slots), else -1 */
    int32_t reserved;  /* 0 */
    uint64_t expected; /* signal value it waited for */
    uint64_t observed; /* last value it read; expected - observed are missing */
} rr_error_record_t;

typedef void *rr_stream_t; /* a hipStream_t; NULL is the null stream */

/* ------------------------------------------------------------ collectives */

/* AllReduce (sections 1 and 4-6 of the loosp.cn post).  In place: bufs is a host
   array of R device pointers, each to `count` elements of `dt`, 16-byte aligned,
   pairwise disjoint, on the current device.  Afterwards every bufs[r] holds the
   reduction described above.  R == 1 or count == 0 is a no-op.
   Errors: RR_ERR_INVALID (R outside 1..64, nslices outside 1..1024, NULL or
   misaligned or overlapping buffers, a buffer not inside one device allocation,
   unknown dtype or op), RR_ERR_UNSUPPORTED (a persistent mode was requested but
   the grid cannot be resident), RR_ERR_HIP, RR_ERR_NOMEM. */
rr_status_t allreduce_ring(void *const *bufs, int R, size_t count, rr_dtype_t dt, rr_op_t op,
                           int nslices, rr_stream_t stream);

/* ReduceScatter (section 5).  In place, arguments as allreduce_ring.  Afterwards
   chunk (r + 1) mod R of bufs[r] holds the finished reduction of that chunk, and
   chunk c of bufs[r] holds the ring's partial fold of ranks c, c+1, ..., r (for
   c == r: rank r's own input, untouched). */
rr_status_t reduce_scatter_ring(void *const *bufs, int R, size_t count, rr_dtype_t dt,
                                rr_op_t op, int nslices, rr_stream_t stream);

/* AllGather (section 6).  In place, arguments as allreduce_ring without an op.
   Before: chunk (r + 1) mod R of bufs[r] holds the data to spread.  Afterwards
   chunk c of every buffer is a bitwise copy of chunk c of bufs[(c - 1) mod R]. */
rr_status_t all_gather_ring(void *const *bufs, int R, size_t count, rr_dtype_t dt, int nslices,
                            rr_stream_t stream);

/* The same three with explicit options (opt may be NULL for the defaults). */
rr_status_t allreduce_ring_ex(void *const *bufs, int R, size_t count, rr_dtype_t dt, rr_op_t op,
                              int nslices, const rr_options_t *opt, rr_stream_t stream);
rr_status_t reduce_scatter_ring_ex(void *const *bufs, int R, size_t count, rr_dtype_t dt,
                                   rr_op_t op, int nslices, const rr_options_t *opt,
                                   rr_stream_t stream);
rr_status_t all_gather_ring_ex(void *const *bufs, int R, size_t count, rr_dtype_t dt,
                               int nslices, const rr_options_t *opt, rr_stream_t stream);

/* allreduce_ring_ex with a clock stamp per hop: the tracing of the ring's own
   hops (where a hop's time goes: waiting for its hand-off, moving its data; how
   far apart the ranks finish the same hop), as counting_barrier_run_timed does
   for the barrier alone.  `stamps` is caller-owned device memory of at least
   nslices * team * R * 2(R-1) * 3 uint64 words (team as rr_plan_query reports
   it), 8-byte aligned; `stamp_words` is its length.  For lane l (= slice *
   team + member), rank r and hop g (1 .. 2(R-1)), the three words at
   ((l * R + r) * 2(R-1) + g - 1) * 3 receive the device's constant-rate wall
   clock when the rank's workgroup starts waiting for the hop's hand-off, when
   the wait is over and the data movement begins, and when the hop's arrival
   has been sent (for the last hop: when its stores were issued).  The first
   hop has no wait (its first two words are two clock reads in a row).  *clock_khz receives the clock's
   rate (host pointer).  Stamps of hops a failed wait skipped stay as they
   were.  The call allocates nothing beyond allreduce_ring_ex.  Errors: as
   allreduce_ring_ex, plus RR_ERR_INVALID for a null or misaligned `stamps`, a
   null `clock_khz`, too few words, or (unless RR_FLAG_NO_POINTER_CHECK) a
   stamps range outside one device allocation. */
rr_status_t allreduce_ring_timed(void *const *bufs, int R, size_t count, rr_dtype_t dt,
                                 rr_op_t op, int nslices, const rr_options_t *opt,
                                 uint64_t *stamps, size_t stamp_words, uint32_t *clock_khz,
                                 rr_stream_t stream);

/* ------------------------------------------------- the staged, out-of-place loop */

/* AllReduce as the staged primitives of Table V (the loosp.cn post, sections
   8-10): at step k rank r handles chunk (r - k) mod R -- step 0 send, steps
   1..R-2 recvReduceSend, step R-1 recvReduceCopySend, steps R..2R-3
   recvCopySend, step 2R-2 recv.  Out of place: sendbufs[r] (count elements) is
   only read; recvbufs[r] receives the result, the same bits as allreduce_ring
   (same chunks, same fold order).  recvbufs[r] == sendbufs[r] is allowed (in
   place); any other overlap is not.  Messages travel through library-owned
   receive buffers of two chunk-sized slots per rank (2 * count elements in
   all, allocated on first use and grown on demand, outgrown ones kept until
   rr_finalize; not under stream capture),
   handed off by a `ready` signal per (lane, rank) and returned by a `credit`
   signal, so traffic is (6R - 4) * count * elem bytes instead of the in-place
   ring's 5(R - 1).  Options: sync AUTO, P2P or LAUNCH (BARRIER is
   RR_ERR_UNSUPPORTED), team, timeout_ns, inject, flags; block must be 0 or 512.
   Errors: as allreduce_ring, plus RR_ERR_INVALID for overlapping buffers. */
rr_status_t allreduce_ring_staged(const void *const *sendbufs, void *const *recvbufs, int R,
                                  size_t count, rr_dtype_t dt, rr_op_t op, int nslices,
                                  const rr_options_t *opt, rr_stream_t stream);

/* allreduce_ring_staged for callers that cannot allocate device memory: code
   under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
   Same arguments, options, results (the same bits) and errors as
   allreduce_ring_staged, but it never allocates: the receive slots, signals,
   shadows and failure record live in a static device array of this library
   (about 65 MiB on every device the library runs on, held until the process
   ends), which every call on a device shares.  Limits: the receive slots hold
   64 MiB, i.e. 2 * R * chunk bytes <= 64 MiB with chunk = ceil(count / R)
   rounded up to a 16-byte vector (about count * elem <= 32 MiB), and a plan may
   use at most 4096 (lane, rank) signal pairs (R * nslices <= 4096; the team is
   chosen within it).  Beyond either limit the call returns RR_ERR_UNSUPPORTED
   before enqueuing anything.  Calls that overlap in time on one device race on
   the shared array: issue them on one stream or order them.  A wait that timed
   out is reported by rr_last_kernel_error like any other, which allocates
   nothing either. */
rr_status_t allreduce_ring_staged_noalloc(const void *const *sendbufs, void *const *recvbufs,
                                          int R, size_t count, rr_dtype_t dt, rr_op_t op,
                                          int nslices, const rr_options_t *opt,
                                          rr_stream_t stream);

/* ReduceScatter with the standalone collective's numbering (the loosp.cn post,
   section 2: which rank keeps which reduced chunk is a matter of numbering).
   sendbufs[r] holds R blocks of recvcount elements, block q at element
   q * recvcount; recvbufs[r] (recvcount elements) receives block r reduced
   over all ranks, folded around the ring from rank r+1: the staged loop
   shifted by one chunk (send, recvReduceSend x (R-2), recvReduceCopy).  Any
   recvcount; buffers 16-byte aligned and pairwise disjoint.  Traffic
   (3R - 1) * R * recvcount * elem bytes.  Options and errors as
   allreduce_ring_staged. */
rr_status_t reduce_scatter(const void *const *sendbufs, void *const *recvbufs, int R,
                           size_t recvcount, rr_dtype_t dt, rr_op_t op, int nslices,
                           const rr_options_t *opt, rr_stream_t stream);

/* AllGather (the loosp.cn post, section 3): sendbufs[r] holds sendcount
   elements; recvbufs[r] receives R blocks, block q = sendbufs[q], bit for bit
   (copySend, recvCopySend x (R-2), recv).  Any sendcount; buffers 16-byte
   aligned and pairwise disjoint.  Traffic (3R - 1) * R * sendcount * elem
   bytes.  Options and errors as allreduce_ring_staged. */
rr_status_t all_gather(const void *const *sendbufs, void *const *recvbufs, int R,
                       size_t sendcount, rr_dtype_t dt, int nslices, const rr_options_t *opt,
                       rr_stream_t stream);

/* ---------------------------------------------------------------- AlltoAll */

/* The pure AlltoAll of the 2kiu.com article on NCCL GIN (section "a pure GIN
   AlltoAll kernel"): sendbufs[r] and recvbufs[r] hold R blocks of `count`
   elements; afterwards block r of recvbufs[q] is block q of sendbufs[r], bit
   for bit.  Each workgroup puts its part of rank r's R blocks and then adds 1
   to every receiver's counting signal; one workgroup per receiver waits for
   all R * parts arrivals (R when a block is one part), advancing a persisted
   shadow, so the signal never needs a reset or an entry barrier.  Buffers
   16-byte aligned and pairwise disjoint; any count.  Traffic 2 * R * R * count
   * elem bytes.  Options: timeout_ns, inject, flags (sync AUTO or P2P).
   Errors: RR_ERR_INVALID (bad sizes, NULL, misaligned or overlapping
   buffers), RR_ERR_UNSUPPORTED (grid not resident), RR_ERR_HIP. */
rr_status_t alltoall(const void *const *sendbufs, void *const *recvbufs, int R, size_t count,
                     rr_dtype_t dt, const rr_options_t *opt, rr_stream_t stream);

/* The plan a call with these arguments would run; no device work.  `phase` is
   0 for AllReduce, 1 for ReduceScatter, 2 for AllGather (the in-place ring),
   3 for allreduce_ring_staged, 4 for reduce_scatter (count = recvcount), 5 for
   all_gather (count = sendcount), 6 for alltoall (count per block; team =
   parts per block).  Errors as the call. */
rr_status_t rr_plan_query(int R, size_t count, rr_dtype_t dt, int nslices, int phase,
                          const rr_options_t *opt, rr_plan_t *out);

/* ------------------------------------------------------- counting barrier */

/* A standalone set of counting signals: `ncontexts` contexts of `nwaiters`
   waiters, one 64-bit signal and one shadow each (DeepEP pull request, section
   "Fix": one signal per waiter whatever the team size), plus, for comparison,
   the per-peer layout that pull request replaced: a row of nwaiters slots and
   shadows per waiter.  Caller-owned; lives in device memory of the current
   device: about ncontexts * nwaiters * (144 + 16 * round_up(nwaiters, 16)) bytes,
   plus one signal and shadow per context for the shared layout
   (RR_FLAG_SHARED_SIGNAL). */
typedef struct rr_counting_barrier rr_counting_barrier_t;

/* Errors: RR_ERR_INVALID (nwaiters outside 1..64, ncontexts outside 1..1024,
   out NULL), RR_ERR_NOMEM, RR_ERR_HIP. */
rr_status_t counting_barrier_create(int nwaiters, int ncontexts, rr_counting_barrier_t **out);

/* Frees the object; waits for its device work first.  NULL is a no-op. */
rr_status_t counting_barrier_destroy(rr_counting_barrier_t *b);

/* Zeroes every signal and shadow, ordered on `stream`.  Only while no kernel
   uses the barrier: a reset must not race other updates (2kiu.com article on
   NCCL GIN, section "Signal methods"). */
rr_status_t counting_barrier_reset(rr_counting_barrier_t *b, rr_stream_t stream);

/* Presets every signal and shadow to `value` (wrap tests); quiescent only. */
rr_status_t counting_barrier_preset(rr_counting_barrier_t *b, uint64_t value, rr_stream_t stream);

/* Reads one waiter's signal and shadow, synchronously (waits for the device):
   the signal's current value, as the read method of the 2kiu.com article on NCCL
   GIN (section "Signal methods") returns it, and the shadow the waiter keeps.
   waiter -1 reads the context's shared signal (RR_FLAG_SHARED_SIGNAL) and its
   shadow.  Errors: RR_ERR_INVALID (b NULL, ctx or waiter out of range),
   RR_ERR_HIP. */
rr_status_t counting_barrier_read(rr_counting_barrier_t *b, int ctx, int waiter, uint64_t *value,
                                  uint64_t *shadow);

/* Reads the per-peer slot of `peer` in `waiter`'s row and the waiter's shadow
   of it, synchronously.  Errors: RR_ERR_INVALID (indices out of range or
   peer == waiter), RR_ERR_HIP. */
rr_status_t counting_barrier_read_peer(rr_counting_barrier_t *b, int ctx, int waiter, int peer,
                                       uint64_t *value, uint64_t *shadow);

/* Steps that `waiter` passed, in audited counting runs (RR_FLAG_AUDIT) since
   the last reset, before every peer's arrival for that step had reached it: a
   stand-in from a peer one step ahead completed its count.  Synchronous.
   Errors: RR_ERR_INVALID, RR_ERR_HIP. */
rr_status_t counting_barrier_early_passes(rr_counting_barrier_t *b, int ctx, int waiter,
                                          uint64_t *count);

/* Runs `nsteps` barrier steps over the first `ncontexts` contexts with R
   waiters each, one workgroup per (context, waiter), in one kernel: the counting
   barrier of the DeepEP pull request (section "Fix": every peer adds 1 to the
   waiter's one signal, the waiter advances its shadow by the expected arrivals
   and polls that signal), or, for comparison, the layouts below.  Per step a
   waiter arrives (opt->sync RR_SYNC_BARRIER or AUTO: adds 1 to every other
   waiter's signal in its context, or with RR_FLAG_SHARED_SIGNAL to the
   context's one signal; RR_SYNC_P2P: adds 1 to its successor's;
   RR_SYNC_PER_PEER: adds 1 to its own slot in every other waiter's row) and
   then advances its shadow by `expected_per_step` and waits for its own signal
   (shared: the context's; per peer: advances every slot's shadow by it and
   waits for every slot).  The right expectation is R-1 (barrier), R (shared)
   or 1 (p2p, per peer); a larger one
   times out (RR_ERR_TIMEOUT from rr_last_kernel_error, with the missing count;
   per peer also with the missing peer).  With nsteps == 0 it launches the same
   kernel doing nothing, to time the launch.
   Errors: RR_ERR_INVALID (R > nwaiters, ncontexts > the object's, nsteps < 0),
   RR_ERR_UNSUPPORTED (grid cannot be resident), RR_ERR_HIP. */
rr_status_t counting_barrier_run(rr_counting_barrier_t *b, int R, int nsteps, int ncontexts,
                                 uint64_t expected_per_step, const rr_options_t *opt,
                                 rr_stream_t stream);

/* counting_barrier_run, with the in-kernel step times that the per-step latency
   is read from (the latency measurement the DeepEP pull request's "Performance"
   section makes for the network barrier, here taken on the device).  `stamps`
   is caller-owned device memory of ncontexts * R * (nsteps + 1) uint64 words,
   8-byte aligned; for context c and waiter q, word (c * R + q) * (nsteps + 1)
   receives the device's constant-rate wall clock before that waiter's first
   step, and word ... + k the clock when its wait for step k was over (k =
   1..nsteps).  *clock_khz receives that clock's rate (host pointer).  One clock
   serves the whole device, so stamps of different waiters compare directly.
   Stamps of a waiter whose wait failed stay as they were.  The call allocates
   nothing.  Errors: as counting_barrier_run, plus RR_ERR_INVALID for a null or
   misaligned `stamps`, a null `clock_khz` or, unless RR_FLAG_NO_POINTER_CHECK,
   a `stamps` range outside one device allocation. */
rr_status_t counting_barrier_run_timed(rr_counting_barrier_t *b, int R, int nsteps,
                                       int ncontexts, uint64_t expected_per_step,
                                       const rr_options_t *opt, uint64_t *stamps,
                                       uint32_t *clock_khz, rr_stream_t stream);

/* ---------------------------------------------------------------- support */

/* Waits for `stream`, then reports and clears the device's failure record (that
   of the library-owned workspace, else that of allreduce_ring_staged_noalloc's
   static array; it allocates nothing): the
   timeout diagnostic of the DeepEP pull request (section "Cost": how many of the
   expected arrivals are missing, and at which signal).
   Returns RR_OK if no wait failed since the last call, else the recorded status
   (RR_ERR_TIMEOUT) with the record in *rec (rec may be NULL).  While a failure
   is recorded every ring and barrier kernel on the device returns at once
   without touching data (sticky), so check after a call whose results matter.
   Clearing also resets the ring workspace's signals and shadows. */
rr_status_t rr_last_kernel_error(rr_stream_t stream, rr_error_record_t *rec);

/* Creates the current device's workspace now (so that later calls allocate
   nothing), and looks up the device address of allreduce_ring_staged_noalloc's
   static array.  Errors: RR_ERR_HIP, RR_ERR_NOMEM. */
rr_status_t rr_init(void);

/* Presets every ring-workspace signal and shadow of the current device to
   `value`, ordered on `stream` (tests of the rolling comparison near 2^64). */
rr_status_t rr_workspace_preset(uint64_t value, rr_stream_t stream);

/* Copies `bytes` bytes from src to dst (device pointers, 16-byte aligned, not
   overlapping) with the library's streaming copy kernel: the bandwidth
   reference and counter calibration for the ring kernels.  Errors:
   RR_ERR_INVALID, RR_ERR_HIP. */
rr_status_t rr_hbm_copy(void *dst, const void *src, size_t bytes, rr_stream_t stream);

/* Human-readable name of a status. */
const char *rr_status_string(rr_status_t s);

/* RR_ABI_VERSION of the loaded library. */
int rr_abi_version(void);

/* Frees every device's workspace (and the staged loop's receive buffers).  No
   call may be in flight, and a graph captured before must not be replayed after:
   its launches hold the freed addresses.  The next call on a device creates a
   fresh workspace, as the first one did. */
void rr_finalize(void);

#ifdef __cplusplus
}
#endif

#endif /* RR_H */
