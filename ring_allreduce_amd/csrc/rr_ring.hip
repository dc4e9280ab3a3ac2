// rr_ring.hip -- ring AllReduce over virtual ranks on one MI355X: kernels and
// the C ABI declared in include/rr.h.
//
// Method (post "Why AllReduce = ReduceScatter + AllGather -- with NCCL Ring
// AllReduce", loosp.cn, sections 4-6): global hop g = 1 .. 2(R-1).  Hops 1..R-1
// are the ReduceScatter rounds: rank r folds chunk (r - g + 1) mod R of its own
// buffer (the partial it received last round, or its input in round 1) into the
// same chunk of its successor's buffer.  Hops R..2R-2 are the AllGather rounds
// t = g - (R-1): rank r copies chunk (r + 2 - t) mod R into its successor's
// buffer.  Rank r's hop g needs only rank r-1's hop g-1 (its data), and every
// earlier reader of what it overwrites is an ancestor of that chain, so a
// predecessor hand-off per hop is all the ordering the ring needs.
//
// Work decomposition: chunk -> `nslices` slices -> `team` sub-ranges.  A lane is
// one (slice j, member w) pair; workgroup (r, lane) owns that sub-range for rank
// r in every chunk, so its hop-g input was written by workgroup (r-1, lane) at
// hop g-1.  Every lane is an independent context with one 64-bit signal per
// rank: after each hop the producer adds 1 to its successor's signal and the
// consumer advances its shadow by 1 and waits (P2P); or, for a per-hop barrier,
// every workgroup of the lane adds 1 to all R-1 other ranks' signals and each
// waiter advances its shadow by R-1 (the counting barrier of the DeepEP pull
// request "make the rail barrier a counting barrier", section "Fix").
//
// One producer per rank per signal is what makes the count safe to hand data
// over.  Had the W workgroups of a slice shared one signal, a workgroup running
// a hop ahead could supply the increment of a teammate that has not finished --
// the hazard the same pull request describes for anonymous counting (section
// "Scoped to the rail team": a count says that enough arrived, not who) -- and
// the consumer of that teammate's sub-range would read stale data.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "rr.h"
#include "rr_device.hpp"

namespace rr {

constexpr int kMaxDevices = 64;
constexpr int kMaxDepth = 4;
constexpr int kSlots = RR_MAX_SLICES * RR_MAX_RANKS;  // (context, rank) pairs
constexpr uint64_t kDefaultTimeoutNs = 2000000000ull;
// Bytes one hop of the lanes in flight may move (3 N / rounds over all ranks):
// fewer keep a partial cached until the next hop reads it, more save hand-offs.
// Predecessor hand-offs: max(96 MiB, 12 MiB x R), one lane per workgroup.  A
// long ring (16 ranks or more) whose hop moves at least 384 MiB over all ranks
// interleaves two lanes per workgroup instead, with 384 MiB in flight.  A
// barrier per hop waits for all R ranks of a lane and prefers fewer, larger
// rounds: 48 MiB x R, within [192, 384] MiB, two lanes per workgroup.  Fitted on
// MI355X to two sweeps of R = 2..64 x 32 MiB..1 GiB per rank (56 cases, depth 1
// and 2, rounds 1..64): 1.5% slower than the best plan of each case on average,
// against 2.4% for the earlier budget (max(96 MiB, 12 MiB x R), doubled for the
// barrier; one lane per workgroup without one), which lost 8-13% at 64 ranks x
// 256 MiB and 5-8% with predecessor hand-offs at 16 ranks x 128 MiB..1 GiB.
constexpr uint64_t kRoundBytesMin = 96ull << 20;
constexpr uint64_t kRoundBytesPerRank = 12ull << 20;
constexpr uint64_t kWideHopBytes = 384ull << 20;
constexpr uint64_t kWideRoundBytes = 384ull << 20;
constexpr uint64_t kBarrierRoundPerRank = 48ull << 20;
constexpr uint64_t kBarrierRoundMin = 192ull << 20;
constexpr uint64_t kBarrierRoundMax = 384ull << 20;
// The staged loop bounds one step of the lanes in flight the same way: 192 MiB
// for its AllReduce and ReduceScatter (a sweep of R = 2..64, 512 MiB..4 GiB:
// 1.2% and 0.5% from the best power-of-two rounds on average).  Its AllGather
// only forwards data, and its hand-offs stay in the L2s when a step moves
// max(48 MiB, 384 MiB / R) over all ranks (2.2% from the best on average, against
// 7% with 192 MiB; 9% faster at 8 ranks x 64 MiB, 15% at 64 ranks x 32 MiB).
constexpr uint64_t kStagedRoundBytes = 192ull << 20;
constexpr uint64_t kGatherRoundMin = 48ull << 20;
constexpr uint64_t kGatherRoundSpan = 384ull << 20;
constexpr uint64_t kLongNapBytes = 64ull << 20;
// The Infinity Cache: above this footprint the ring's loads of the
// predecessor's buffer are non-temporal.
constexpr uint64_t kInfinityCacheBytes = 256ull << 20;
// Lanes a workgroup interleaves when the caller does not choose: a per-hop
// barrier waits for the slowest of R workgroups, which a second lane hides; a
// predecessor hand-off is cheap enough that a second lane costs more than it
// hides, except on a long ring moving a wide hop (see the rounds budget above;
// measured on MI355X).
constexpr int kAutoDepthBarrier = 2;
constexpr int kAutoDepthP2P = 1;
constexpr int kAutoDepthWide = 2;
// Workgroup size when the caller does not choose.  Columns are planned for
// 512-thread workgroups (two per CU); the threads per workgroup then follow the
// lane piece (the bytes one workgroup moves per lane and hop):
//   at most 2 KiB (a latency-bound call)                          128 threads
//   16-32 KiB                                                      256
//   at most 64 KiB on a long ring (16 ranks or more) over buffers
//   larger than the Infinity Cache                                 128
//   otherwise                                                      512
// A workgroup's hop ends when its slowest wave's stores have drained, and along
// a long chain of hand-offs those tails add up, so fewer waves per workgroup pay
// when a piece is small; a piece of 64 KiB or more on a shorter ring streams
// better with 512.  Fitted on MI355X to 90 cases at fixed columns (R = 4..64,
// 4 KiB..256 MiB per rank, both modes, 128 / 256 / 512 threads): 0.6% slower than
// the best size of each case on average (worst 9%, pieces of 4-16 KiB, where no
// size wins consistently), against 4.2% (worst 31%) for 512 everywhere but the
// long-ring rule.
constexpr int kAutoBlock = 512;
constexpr int kSmallBlock = 128;
constexpr int kMidBlock = 256;
constexpr uint64_t kTinyPieceBytes = 2ull << 10;
constexpr uint64_t kMidPieceLo = 16ull << 10;   // exclusive
constexpr uint64_t kMidPieceHi = 32ull << 10;
constexpr int kLongRingRanks = 16;
constexpr uint64_t kLongRingPieceBytes = 64ull << 10;

// Per-launch tag of the XCD table, kept on the device so that a launch replayed
// from a captured graph still gets a fresh one: every workgroup reads `gen` at
// start, and the last workgroup to leave a launch advances it for the next
// launch (launches on one device are ordered, so no launch starts before the
// previous one has left).  Zero is never used: the table starts zeroed.
struct LaunchTag {
    uint64_t* gen;    // current tag, in [1, 2^32)
    uint64_t* exits;  // workgroups of the running launch that have left
};

struct RingArgs {
    void* bufs[RR_MAX_RANKS];
    uint64_t count;      // elements per rank
    uint64_t chunk_len;  // nominal chunk length (elements, vector multiple)
    uint64_t slice_len;  // nominal slice length
    uint64_t sub_len;    // nominal length per team member
    uint64_t* sig;       // signal of slot s at sig[s * kSignalStride]
    uint64_t* shadow;    // shadow of slot s
    uint64_t* xcc_table; // per workgroup: (generation << 8) | XCC id, published at start
    ErrorRecord* err;
    uint64_t timeout_ticks;
    LaunchTag launch;    // per-launch tag of the XCD table (device side)
    int32_t fuse;        // 1: fused boundary (the last ReduceScatter hop also does the first AllGather hop)
    int32_t R;
    int32_t team;
    int32_t g_first;     // hops run by this launch, 1-based, inclusive
    int32_t g_last;
    int32_t sync;        // SYNC_NONE (one hop per launch), SYNC_P2P, SYNC_BARRIER
    int32_t xcd_map;
    uint32_t inject;
    int32_t cols;        // workgroups per rank = grid / R
    int32_t rounds;      // lane groups each workgroup runs one after another
    int32_t depth;       // lanes each workgroup interleaves hop by hop (1..kMaxDepth)
    int32_t long_nap;    // barrier waits poll slowly (a hop moves enough data to hide it)
    int32_t stream_in;   // loads of the predecessor's buffer are non-temporal
};

__device__ __forceinline__ uint64_t umin(uint64_t a, uint64_t b) { return a < b ? a : b; }

__device__ __forceinline__ uint32_t launch_generation(const LaunchTag& t) {
    return (uint32_t)__hip_atomic_load(t.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by every workgroup once, after all of its work (every exit path).
__device__ __forceinline__ void leave_launch(const LaunchTag& t) {
    if (threadIdx.x != 0) return;
    const uint64_t before =
        __hip_atomic_fetch_add(t.exits, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (before + 1 != (uint64_t)gridDim.x) return;
    uint32_t next = launch_generation(t) + 1;
    if (next == 0) next = 1;
    __hip_atomic_store(t.exits, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(t.gen, (uint64_t)next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int wrap(int a, int m) {
    const int r = a % m;
    return r < 0 ? r + m : r;
}

// Workgroups are dealt to the 8 XCDs round-robin by index.  Both kernels lay
// their grid out as columns of R workgroups (one per rank) with every column on
// one XCD: block b = ((col / 8) * R + rank) * 8 + col % 8.  Column counts are
// padded to a multiple of 8; padding columns exit at once.
struct Place {
    int rank;
    int col;
};

__device__ __forceinline__ Place place_of(int b, int R, bool xcd_map) {
    if (xcd_map) {
        const int x = b & 7, k = b >> 3;
        return {k % R, (k / R) * 8 + x};
    }
    return {b % R, b / R};
}

__device__ __forceinline__ int block_of(int rank, int col, int R, bool xcd_map) {
    return xcd_map ? ((col >> 3) * R + rank) * 8 + (col & 7) : col * R + rank;
}

// The XCD (accelerator complex die) this wave runs on.
__device__ __forceinline__ uint32_t xcc_id() {
    return __builtin_amdgcn_s_getreg(20 /* HW_REG_XCC_ID */ | (0 << 6) | ((4 - 1) << 11));
}

// Every synchronising workgroup publishes (generation << 8) | XCC id at start.
__device__ __forceinline__ void publish_xcc(uint64_t* table, uint32_t generation, uint32_t xcc) {
    __hip_atomic_store(&table[blockIdx.x], ((uint64_t)generation << 8) | xcc, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Called by wave 0.  1 when the R workgroups of column `col` all run on this
// workgroup's XCD (read from the published table), 0 if not; they then share one
// L2, the point where producer stores and consumer loads meet.  All R
// workgroups of the column compute the same answer.  -1 if one never published
// (timeout, or a failure elsewhere).
__device__ int column_on_one_xcd(const uint64_t* table, uint32_t generation, int R, int col,
                                 bool xcd_map, uint32_t mine, const ErrorRecord* err,
                                 uint64_t timeout_ticks) {
    const int k = threadIdx.x;
    int same = 1;
    int failed = 0;
    if (k < R) {
        const uint64_t* e = &table[block_of(k, col, R, xcd_map)];
        uint64_t v = sig_read(e);
        const uint64_t start = wall_clock64();
        uint32_t spins = 0;
        while ((uint32_t)(v >> 8) != generation) {
            __builtin_amdgcn_s_sleep(1);
            v = sig_read(e);
            if ((++spins & 31u) == 0u &&
                (sig_read(&err->flag) != 0 || wall_clock64() - start > timeout_ticks)) {
                failed = 1;
                break;
            }
        }
        same = !failed && (uint32_t)(v & 0xFFu) == mine;
    }
    if (__any(failed)) return -1;
    return __all(same) ? 1 : 0;
}

// Producer side of a hand-off, executed by every thread of the workgroup
// before its barrier and arrival.  Same XCD: each wave waits until its stores
// have reached the shared L2.  Otherwise, also write the L2 back so that other
// XCDs see the stores -- once per workgroup, after every wave's stores are in L2.
__device__ __forceinline__ void release_stores(bool local) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!local) {
        __syncthreads();
        if (threadIdx.x < 64) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    }
}

// Consumer side, executed by the one thread that saw the signal, before the
// workgroup barrier.  Same XCD: nothing to invalidate -- incoming data are read
// with device-scope loads that skip the L1 and meet the producer's stores in the
// shared L2 (a workgroup-scope L1 invalidate would not do: outside
// thread-group-split mode the L1 counts as coherent for one workgroup and is left
// alone).  Otherwise: an agent-scope acquire (L1 and L2 invalidate), completed
// before any wave loads.
__device__ __forceinline__ void acquire_stores(bool local) {
    if (local) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    } else {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
}

// Loads of the incoming buffer -- data another workgroup wrote earlier in this
// launch -- go through a buffer descriptor with device-scope coherence (sc1):
// they skip this CU's L1, which may still hold lines of the same addresses from
// an earlier hop (a workgroup reads a chunk's partial in ReduceScatter and its
// finished value one AllGather hop later), and are served by the L2.  Within one
// XCD that L2 already holds the producer's stores, so the consumer needs no
// cache invalidation at all.  The descriptor also bounds every load: a load
// outside [base, base + bytes) returns zero instead of touching memory.
//
// When the R buffers together exceed the Infinity Cache, the in-place ring also
// marks these loads non-temporal (nt): a partial or a finished chunk read from
// the predecessor's buffer is not read again before it is overwritten, so its
// lines are the first the caches should give up, which keeps the lines a rank
// writes for its own successor cached until the next hop reads them (measured:
// 4% at 8 ranks x 64 MiB, 12% at 64 ranks x 32 MiB in barrier mode).  When
// everything fits, the hint only evicts lines that would have hit (up to 30%
// slower at 16 ranks x 16 MiB), so those calls keep device scope alone.  The
// staged loop's receive slots are rewritten every other step and lose 2-5% with
// the hint, so they never use it.
constexpr int kAuxDeviceScope = 16;             // sc1
constexpr int kAuxNonTemporal = 2;              // nt
constexpr int kAuxRingIncoming = kAuxDeviceScope | kAuxNonTemporal;
constexpr int kAuxStoreOut = kAuxDeviceScope | kAuxNonTemporal;  // AlltoAll puts
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw (untyped) buffer access on gfx9
constexpr uint64_t kPieceBytes = 1ull << 30;    // one descriptor covers at most this

__device__ __forceinline__ __amdgpu_buffer_rsrc_t incoming(const void* base, uint64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             (int)kBufferWord3);
}

template <int AUX = kAuxDeviceScope>
__device__ __forceinline__ u32x4 load_in(__amdgpu_buffer_rsrc_t rs, uint32_t vec) {
    return __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(vec * 16u), 0, AUX));
}

// One hop of one workgroup over elements [lo, hi) of both buffers.  ReduceScatter:
// dst = fold(src, dst).  AllGather: dst = src, bit for bit.  16-byte vectors,
// U vectors per thread in flight, then a scalar tail (only at the ragged end).
template <int DT, int OP, int BLOCK, int U, int AUX>
__device__ __forceinline__ void hop_piece(bool reduce, const void* srcbuf, void* dstbuf,
                                          void* dst2buf, uint64_t lo, uint64_t hi) {
    constexpr int ES = ElemBytes<DT>::value;
    constexpr int V = 16 / ES;
    const uint64_t n = hi - lo;
    const uint32_t nv = (uint32_t)(n / V);
    const char* sb = (const char*)srcbuf + lo * ES;
    const __amdgpu_buffer_rsrc_t rs = incoming(sb, n * ES);
    u32x4* __restrict__ d = (u32x4*)((char*)dstbuf + lo * ES);
    u32x4* d2 = dst2buf ? (u32x4*)((char*)dst2buf + lo * ES) : nullptr;
    uint32_t i = threadIdx.x;
    if (reduce && d2) {
        // recvReduceCopySend: the finished chunk goes to the owner's buffer and on
        // to the owner's successor in the same pass
        for (; i + (U - 1) * BLOCK < nv; i += U * BLOCK) {
            u32x4 x[U], y[U];
#pragma unroll
            for (int u = 0; u < U; ++u) x[u] = load_in<AUX>(rs, i + u * BLOCK);
#pragma unroll
            for (int u = 0; u < U; ++u) y[u] = d[i + u * BLOCK];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const u32x4 v = fold4<DT, OP>(x[u], y[u]);
                d[i + u * BLOCK] = v;
                d2[i + u * BLOCK] = v;
            }
        }
        for (; i < nv; i += BLOCK) {
            const u32x4 v = fold4<DT, OP>(load_in<AUX>(rs, i), d[i]);
            d[i] = v;
            d2[i] = v;
        }
    } else if (reduce) {
        for (; i + (U - 1) * BLOCK < nv; i += U * BLOCK) {
            u32x4 x[U], y[U];
#pragma unroll
            for (int u = 0; u < U; ++u) x[u] = load_in<AUX>(rs, i + u * BLOCK);
#pragma unroll
            for (int u = 0; u < U; ++u) y[u] = d[i + u * BLOCK];
#pragma unroll
            for (int u = 0; u < U; ++u) d[i + u * BLOCK] = fold4<DT, OP>(x[u], y[u]);
        }
        for (; i < nv; i += BLOCK) d[i] = fold4<DT, OP>(load_in<AUX>(rs, i), d[i]);
    } else {
        constexpr int UC = 2 * U;
        for (; i + (UC - 1) * BLOCK < nv; i += UC * BLOCK) {
            u32x4 x[UC];
#pragma unroll
            for (int u = 0; u < UC; ++u) x[u] = load_in<AUX>(rs, i + u * BLOCK);
#pragma unroll
            for (int u = 0; u < UC; ++u) d[i + u * BLOCK] = x[u];
        }
        for (; i < nv; i += BLOCK) d[i] = load_in<AUX>(rs, i);
    }
    const uint64_t t = (uint64_t)nv * V + threadIdx.x;  // fewer than V elements remain
    if (t < n) {
        char* dp = (char*)dstbuf + (lo + t) * ES;
        const int off = (int)(t * ES);
        char* dp2 = dst2buf ? (char*)dst2buf + (lo + t) * ES : nullptr;
        if constexpr (ES == 2) {
            const uint16_t in =
                __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, AUX);
            const uint16_t v =
                reduce ? (uint16_t)Fold<DT, OP>::half(in, *(const uint16_t*)dp) : in;
            *(uint16_t*)dp = v;
            if (dp2) *(uint16_t*)dp2 = v;
        } else {
            const uint32_t in = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, AUX);
            const uint32_t v = reduce ? Fold<DT, OP>::lane(in, *(const uint32_t*)dp) : in;
            *(uint32_t*)dp = v;
            if (dp2) *(uint32_t*)dp2 = v;
        }
    }
}

template <int DT, int OP, int BLOCK, int U>
__device__ __forceinline__ void hop_body(bool reduce, bool stream, const void* srcbuf,
                                         void* dstbuf, void* dst2buf, uint64_t lo, uint64_t hi) {
    constexpr uint64_t kPiece = kPieceBytes / ElemBytes<DT>::value;  // elements, vector multiple
    for (uint64_t p = lo; p < hi; p += kPiece) {
        const uint64_t q = umin(p + kPiece, hi);
        if (stream)
            hop_piece<DT, OP, BLOCK, U, kAuxRingIncoming>(reduce, srcbuf, dstbuf, dst2buf, p, q);
        else
            hop_piece<DT, OP, BLOCK, U, kAuxDeviceScope>(reduce, srcbuf, dstbuf, dst2buf, p, q);
    }
}

template <int DT, int OP, int BLOCK>
__device__ __forceinline__ void ring_body(const RingArgs& a, const uint32_t generation) {
    constexpr int U = 4;
    const int R = a.R;
    const Place pl = place_of(blockIdx.x, R, a.xcd_map != 0);
    const int r = pl.rank, col = pl.col;
    if (col >= a.cols) return;  // padding column
    const int succ = r + 1 == R ? 0 : r + 1;
    const int succ2 = succ + 1 == R ? 0 : succ + 1;
    const bool synced = a.g_last > a.g_first;

    __shared__ int s_stop;
    __shared__ int s_local;
    const uint32_t my_xcc = xcc_id() & 0xFu;
    if (threadIdx.x == 0) {
        s_stop = sig_read(&a.err->flag) != 0;  // a recorded failure is sticky
        if (synced) publish_xcc(a.xcc_table, generation, my_xcc);
    }
    __syncthreads();
    if (s_stop) return;
    // Producer side of the hand-off (release_stores), fixed at the first
    // hand-off of the launch: `local` when all R workgroups of the column run on
    // one XCD and so share its L2.  The consumer side (acquire_stores) is the
    // same either way; its L1 invalidation matters even within one XCD, because a
    // workgroup re-reads a chunk of its incoming buffer (the partial in
    // ReduceScatter, the finished chunk one AllGather hop later).
    bool local = false;
    bool decided = false;
    const uint64_t arrivals = a.sync == SYNC_BARRIER ? (uint64_t)(R - 1) : 1;
    __shared__ int s_stop_lane[kMaxDepth];

    // Lane groups one after another: only cols * depth lanes are in flight at
    // once, so the partial a hop writes is still cached when the next hop reads
    // it, whatever the buffer size.  Within a group the workgroup interleaves its
    // `depth` lanes hop by hop -- hop g of lane 1 runs while lane 0's hand-off
    // for hop g+1 completes.  Every wait targets a (lane, hop) that comes earlier
    // in the (hop, lane) order all workgroups follow, so the interleave cannot
    // deadlock.
    for (int round = 0; round < a.rounds; ++round) {
        int lane[kMaxDepth];
        uint64_t off_lo[kMaxDepth], off_hi[kMaxDepth], shadow[kMaxDepth];
#pragma unroll
        for (int p = 0; p < kMaxDepth; ++p) {
            lane[p] = col + (round * a.depth + p) * a.cols;
            const int j = lane[p] / a.team;
            const int w = lane[p] - j * a.team;
            off_lo[p] = (uint64_t)j * a.slice_len + (uint64_t)w * a.sub_len;
            off_hi[p] = umin(off_lo[p] + a.sub_len,
                             umin((uint64_t)(j + 1) * a.slice_len, a.chunk_len));
            shadow[p] = 0;
            if (p < a.depth && synced && threadIdx.x == 0) shadow[p] = a.shadow[lane[p] * R + r];
        }

        for (int g = a.g_first; g <= a.g_last; ++g) {
#pragma unroll
            for (int p = 0; p < kMaxDepth; ++p) {
                if (p >= a.depth) break;
                const int my_slot = lane[p] * R + r;
                const bool injected = r == 0 && lane[p] == 0;
                if (g > a.g_first) {
                    if (threadIdx.x == 0) {
                        uint64_t target = shadow[p] + arrivals;
                        if ((a.inject & RR_INJECT_EXTRA_EXPECTED) && injected &&
                            g == a.g_first + 1)
                            target += 1;
                        const WaitResult res = sig_wait(&a.sig[(uint64_t)my_slot * kSignalStride],
                                                        target, a.err, a.timeout_ticks,
                                                        a.long_nap != 0);
                        if (res.status == WAIT_TIMEOUT)
                            record_timeout(a.err, lane[p], r, g, target, res.observed);
                        shadow[p] = target;
                        s_stop_lane[p] = res.status != WAIT_OK;
                        acquire_stores(local);
                    }
                    __syncthreads();
                    if (s_stop_lane[p]) return;
                }

                int c;
                bool reduce;
                if (g <= R - 1) {
                    c = wrap(r - g + 1, R);
                    reduce = true;
                } else {
                    c = wrap(r + 2 - (g - (R - 1)), R);
                    reduce = false;
                }
                // Fused boundary: the last ReduceScatter hop also stores the finished
                // chunk in the owner's successor, so the first AllGather hop only
                // passes the hand-off on.
                void* dst2 = a.fuse && g == R - 1 ? a.bufs[succ2] : nullptr;
                const bool skip = a.fuse && g == R;
                const uint64_t base = (uint64_t)c * a.chunk_len;
                const uint64_t lo = base + off_lo[p];
                const uint64_t hi = umin(base + off_hi[p], a.count);
                if (lo < hi && !skip)
                    hop_body<DT, OP, BLOCK, U>(reduce, a.stream_in != 0, a.bufs[r], a.bufs[succ],
                                               dst2, lo, hi);

                if (g < a.g_last) {
                    if (!decided) {
                        if (threadIdx.x < 64) {
                            const int v = column_on_one_xcd(a.xcc_table, generation, R, col,
                                                            a.xcd_map != 0, my_xcc, a.err,
                                                            a.timeout_ticks);
                            if (threadIdx.x == 0) {
                                if (v < 0) record_timeout(a.err, lane[p], r, 0, generation, 0);
                                s_local = v;
                            }
                        }
                        __syncthreads();
                        if (s_local < 0) return;
                        local = s_local == 1;
                        decided = true;
                    }
                    release_stores(local);
                    __syncthreads();
                    const bool drop =
                        (a.inject & RR_INJECT_DROP_ARRIVAL) && injected && g == a.g_first;
                    if (!drop) {
                        if (a.sync == SYNC_BARRIER) {
                            if ((int)threadIdx.x < R - 1) {
                                const int q = wrap(r + 1 + (int)threadIdx.x, R);
                                sig_add(&a.sig[(uint64_t)(lane[p] * R + q) * kSignalStride], 1);
                            }
                        } else if (threadIdx.x == 0) {
                            sig_add(&a.sig[(uint64_t)(lane[p] * R + succ) * kSignalStride], 1);
                        }
                    }
                }
            }
        }
        if (synced && threadIdx.x == 0) {
#pragma unroll
            for (int p = 0; p < kMaxDepth; ++p)
                if (p < a.depth) a.shadow[lane[p] * R + r] = shadow[p];  // sig == shadow again
        }
    }
}

template <int DT, int OP, int BLOCK>
__global__ void __launch_bounds__(BLOCK) ring_kernel(const RingArgs a) {
    ring_body<DT, OP, BLOCK>(a, launch_generation(a.launch));
    leave_launch(a.launch);
}

// ------------------------------------------------------ the staged loop --
//
// The ring as the primitives of one rank (the loosp.cn post, sections 8-10;
// Table V of the paper it discusses), out of place.  Each rank owns a receive
// buffer of kFifoSlots chunk-sized slots per lane; at step k a rank reads the
// message of step k-1 from its own slot (k-1) mod kFifoSlots, combines it with
// its input and/or writes its output, and sends the result into its
// successor's slot k mod kFifoSlots.  Two counting signals per (lane, rank)
// hand the steps off: `ready` (the predecessor's message has landed; one
// arrival per step) and `credit` (the successor has consumed a message, so its
// slot may be written again; one arrival per message).  A sender needs credit
// for message k - kFifoSlots before it writes message k.
//
//   AllReduce       steps 0..2R-2: send, recvReduceSend x (R-2),
//                   recvReduceCopySend, recvCopySend x (R-2), recv; rank r
//                   handles chunk (r - k) mod R at step k.
//   ReduceScatter   the standalone numbering (rank r keeps block r): steps
//                   0..R-1, send, recvReduceSend x (R-2), recvReduceCopy; chunk
//                   (r - k - 1) mod R.
//   AllGather       steps 0..R-1, copySend, recvCopySend x (R-2), recv; chunk
//                   (r - k) mod R.
constexpr int kFifoSlots = 2;
constexpr int kStagedBlock = 512;
// AlltoAll: one 1024-thread workgroup per CU, 8 vectors per thread in flight
// (4 in flight: 2-4% slower at 8 ranks x 64 MiB fp32, bf16 256 MiB and 64 ranks
// x 32 MiB; 256 threads x 8: 3-9% slower)
constexpr int kA2ABlock = 1024;
constexpr int kA2AUnroll = 8;
constexpr int kCopyBlock = 1024;
constexpr int kCopyPerCU = 2;
constexpr int kA2AWavesPerCU = 16;
enum : int { MODE_ALLREDUCE = 0, MODE_RS = 1, MODE_AG = 2 };
enum : int { P_SEND = 0, P_RRS = 1, P_RRCS = 2, P_RCS = 3, P_RECV = 4, P_RRC = 5, P_CS = 6 };

template <int P> struct Prim {
    static constexpr bool in = P != P_SEND && P != P_CS;  // reads the receive slot
    static constexpr bool local = P == P_SEND || P == P_RRS || P == P_RRCS || P == P_RRC || P == P_CS;
    static constexpr bool reduce = P == P_RRS || P == P_RRCS || P == P_RRC;
    static constexpr bool out = P != P_SEND && P != P_RRS;  // writes the output
    static constexpr bool send = P != P_RECV && P != P_RRC;  // writes the successor's slot
};

struct StagedArgs {
    const void* send[kMaxDevices];
    void* recv[kMaxDevices];
    char* fifo;            // R ranks x kFifoSlots slots x slot_len elements
    uint64_t slot_len;     // elements per slot (chunk_len rounded up to a vector)
    uint64_t n;            // AllReduce: elements per rank; else elements per block
    uint64_t chunk_len;    // AllReduce: the partition's chunk length; else n
    uint64_t slice_len;
    uint64_t sub_len;
    uint64_t* ready;
    uint64_t* ready_shadow;
    uint64_t* credit;
    uint64_t* credit_shadow;
    uint64_t* xcc_table;
    ErrorRecord* err;
    uint64_t timeout_ticks;
    LaunchTag launch;
    uint32_t inject;
    int32_t R;
    int32_t team;
    int32_t cols;          // workgroups per rank
    int32_t rounds;        // lane groups each workgroup runs one after another
    int32_t mode;
    int32_t k_first;       // steps this launch runs
    int32_t k_last;
    int32_t xcd_map;
    int32_t aligned;       // every operand 16-byte aligned: the vector path
    int32_t pad;
};

// One step's data over n elements: in (the receive slot, device-scope loads),
// local (the rank's input), out (its output), next (the successor's slot).
// Output stores are non-temporal: nothing in the collective reads them back,
// while the successor reads `next` one step later (measured: 1-3% at 8 ranks).
template <int DT, int OP, int BLOCK, int P>
__device__ __forceinline__ void staged_piece(const void* in, const void* local, void* out,
                                             void* next, uint64_t n, bool aligned) {
    using Q = Prim<P>;
    constexpr int ES = ElemBytes<DT>::value;
    constexpr int V = 16 / ES;
    constexpr int U = 4;
    // (a descriptor of zero bytes when the primitive reads no slot; never used)
    const __amdgpu_buffer_rsrc_t rs = incoming(in, Q::in ? n * ES : 0);
    uint64_t done = 0;
    if (aligned) {
        const uint32_t nv = (uint32_t)(n / V);
        const u32x4* __restrict__ lp = (const u32x4*)local;
        u32x4* __restrict__ op = (u32x4*)out;
        u32x4* __restrict__ np = (u32x4*)next;
        uint32_t i = threadIdx.x;
        for (; i + (U - 1) * BLOCK < nv; i += U * BLOCK) {
            u32x4 x[U], y[U];
            if constexpr (Q::in) {
#pragma unroll
                for (int u = 0; u < U; ++u) x[u] = load_in(rs, i + u * BLOCK);
            }
            if constexpr (Q::local) {
#pragma unroll
                for (int u = 0; u < U; ++u) y[u] = lp[i + u * BLOCK];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                u32x4 v;
                if constexpr (Q::reduce) v = fold4<DT, OP>(x[u], y[u]);
                else if constexpr (Q::in) v = x[u];
                else v = y[u];
                if constexpr (Q::out) __builtin_nontemporal_store(v, &op[i + u * BLOCK]);
                if constexpr (Q::send) np[i + u * BLOCK] = v;
            }
        }
        for (; i < nv; i += BLOCK) {
            u32x4 v;
            if constexpr (Q::reduce) v = fold4<DT, OP>(load_in(rs, i), lp[i]);
            else if constexpr (Q::in) v = load_in(rs, i);
            else v = lp[i];
            if constexpr (Q::out) __builtin_nontemporal_store(v, &op[i]);
            if constexpr (Q::send) np[i] = v;
        }
        done = (uint64_t)nv * V;
    }
    // element by element: the ragged end, or everything when an operand is not
    // 16-byte aligned
    for (uint64_t t = done + threadIdx.x; t < n; t += BLOCK) {
        const int off = (int)(t * ES);
        if constexpr (ES == 2) {
            uint16_t x = 0, y = 0, v;
            if constexpr (Q::in) x = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, kAuxDeviceScope);
            if constexpr (Q::local) y = ((const uint16_t*)local)[t];
            if constexpr (Q::reduce) v = (uint16_t)Fold<DT, OP>::half(x, y);
            else v = Q::in ? x : y;
            if constexpr (Q::out) ((uint16_t*)out)[t] = v;
            if constexpr (Q::send) ((uint16_t*)next)[t] = v;
        } else {
            uint32_t x = 0, y = 0, v;
            if constexpr (Q::in) x = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, kAuxDeviceScope);
            if constexpr (Q::local) y = ((const uint32_t*)local)[t];
            if constexpr (Q::reduce) v = Fold<DT, OP>::lane(x, y);
            else v = Q::in ? x : y;
            if constexpr (Q::out) ((uint32_t*)out)[t] = v;
            if constexpr (Q::send) ((uint32_t*)next)[t] = v;
        }
    }
}

// A piece longer than one buffer descriptor can cover is moved in parts.
template <int DT, int OP, int BLOCK, int P>
__device__ __forceinline__ void staged_move(const char* in, const char* local, char* out, char* next,
                                            uint64_t n, bool aligned) {
    constexpr int ES = ElemBytes<DT>::value;
    constexpr uint64_t kPart = kPieceBytes / ES;
    for (uint64_t p = 0; p < n; p += kPart) {
        const uint64_t m = umin(kPart, n - p);
        staged_piece<DT, OP, BLOCK, P>(in + p * ES, local + p * ES, out + p * ES, next + p * ES, m,
                                       aligned);
    }
}

template <int DT, int OP, int BLOCK>
__device__ __forceinline__ void staged_body(const StagedArgs& a, const uint32_t generation) {
    constexpr int ES = ElemBytes<DT>::value;
    const int R = a.R;
    const Place pl = place_of(blockIdx.x, R, a.xcd_map != 0);
    const int r = pl.rank, col = pl.col;
    if (col >= a.cols) return;  // padding column
    const int succ = r + 1 == R ? 0 : r + 1;
    const int pred = r == 0 ? R - 1 : r - 1;
    const bool synced = a.k_last > a.k_first;
    const int K = a.mode == MODE_ALLREDUCE ? 2 * R - 2 : R - 1;  // last step; steps < K send

    __shared__ int s_stop;
    __shared__ int s_local;
    const uint32_t my_xcc = xcc_id() & 0xFu;
    if (threadIdx.x == 0) {
        s_stop = sig_read(&a.err->flag) != 0;  // a recorded failure is sticky
        if (synced) publish_xcc(a.xcc_table, generation, my_xcc);
    }
    __syncthreads();
    if (s_stop) return;

    bool local = false, decided = false;
    // Lane groups one after another (as in the in-place ring): only the lanes of
    // one round are in flight, so a message is still cached when it is read.
    for (int round = 0; round < a.rounds; ++round) {
    const int lane = col + round * a.cols;
    const int j = lane / a.team, w = lane - j * a.team;
    const uint64_t off_lo = (uint64_t)j * a.slice_len + (uint64_t)w * a.sub_len;
    const uint64_t off_hi =
        umin(off_lo + a.sub_len, umin((uint64_t)(j + 1) * a.slice_len, a.chunk_len));
    const int my_slot = lane * R + r;
    const bool injected = r == 0 && lane == 0;
    uint64_t ready_shadow = 0, credit_base = 0;
    if (synced && threadIdx.x == 0) {
        ready_shadow = a.ready_shadow[my_slot];
        credit_base = a.credit_shadow[my_slot];
    }
    uint64_t credit_target = credit_base;

    for (int k = a.k_first; k <= a.k_last; ++k) {
        const bool has_in = k >= 1, has_send = k < K;
        if (synced) {
            if (threadIdx.x == 0) {
                int stop = 0;
                if (has_in) {  // the predecessor's message of step k-1
                    uint64_t target = ready_shadow + 1;
                    if ((a.inject & RR_INJECT_EXTRA_EXPECTED) && injected && k == 1) target += 1;
                    const WaitResult res = sig_wait(&a.ready[(uint64_t)my_slot * kSignalStride],
                                                    target, a.err, a.timeout_ticks);
                    if (res.status == WAIT_TIMEOUT)
                        record_timeout(a.err, lane, r, k, target, res.observed);
                    ready_shadow = target;
                    stop = res.status != WAIT_OK;
                }
                if (!stop && has_send && k >= kFifoSlots) {  // the successor freed the slot
                    credit_target += 1;
                    const WaitResult res = sig_wait(&a.credit[(uint64_t)my_slot * kSignalStride],
                                                    credit_target, a.err, a.timeout_ticks);
                    if (res.status == WAIT_TIMEOUT)
                        record_timeout(a.err, lane, r, k, credit_target, res.observed, succ);
                    stop = res.status != WAIT_OK;
                }
                if (!stop && has_in) acquire_stores(local);
                s_stop = stop;
            }
            __syncthreads();
            if (s_stop) return;
        }

        const int c = wrap(r - k - (a.mode == MODE_RS ? 1 : 0), R);
        const uint64_t base = a.mode == MODE_ALLREDUCE ? (uint64_t)c * a.chunk_len : 0;
        const uint64_t len = a.mode == MODE_ALLREDUCE
                                 ? (base < a.n ? umin(a.chunk_len, a.n - base) : 0)
                                 : a.n;
        const uint64_t lo = off_lo, hi = umin(off_hi, len);
        if (lo < hi) {
            const char* in = a.fifo + ((uint64_t)(r * kFifoSlots + (k + kFifoSlots - 1) % kFifoSlots) *
                                           a.slot_len + lo) * ES;
            char* next = a.fifo + ((uint64_t)(succ * kFifoSlots + k % kFifoSlots) * a.slot_len + lo) * ES;
            const uint64_t lbase = a.mode == MODE_AG ? 0 : (uint64_t)c * a.chunk_len;
            const uint64_t obase = a.mode == MODE_RS ? 0 : (uint64_t)c * a.chunk_len;
            const char* lp = (const char*)a.send[r] + (lbase + lo) * ES;
            char* op = (char*)a.recv[r] + (obase + lo) * ES;
            const uint64_t m = hi - lo;
            const bool al = a.aligned != 0;
            if (a.mode == MODE_ALLREDUCE) {
                if (k == 0) staged_move<DT, OP, BLOCK, P_SEND>(in, lp, op, next, m, al);
                else if (k < R - 1) staged_move<DT, OP, BLOCK, P_RRS>(in, lp, op, next, m, al);
                else if (k == R - 1) staged_move<DT, OP, BLOCK, P_RRCS>(in, lp, op, next, m, al);
                else if (k < K) staged_move<DT, OP, BLOCK, P_RCS>(in, lp, op, next, m, al);
                else staged_move<DT, OP, BLOCK, P_RECV>(in, lp, op, next, m, al);
            } else if (a.mode == MODE_RS) {
                if (k == 0) staged_move<DT, OP, BLOCK, P_SEND>(in, lp, op, next, m, al);
                else if (k < K) staged_move<DT, OP, BLOCK, P_RRS>(in, lp, op, next, m, al);
                else staged_move<DT, OP, BLOCK, P_RRC>(in, lp, op, next, m, al);
            } else {
                if (k == 0) staged_move<DT, OP, BLOCK, P_CS>(in, lp, op, next, m, al);
                else if (k < K) staged_move<DT, OP, BLOCK, P_RCS>(in, lp, op, next, m, al);
                else staged_move<DT, OP, BLOCK, P_RECV>(in, lp, op, next, m, al);
            }
        }

        if (synced) {
            if (!decided) {
                if (threadIdx.x < 64) {
                    const int v = column_on_one_xcd(a.xcc_table, generation, R, lane,
                                                    a.xcd_map != 0, my_xcc, a.err, a.timeout_ticks);
                    if (threadIdx.x == 0) {
                        if (v < 0) record_timeout(a.err, lane, r, 0, generation, 0);
                        s_local = v;
                    }
                }
                __syncthreads();
                if (s_local < 0) return;
                local = s_local == 1;
                decided = true;
            }
            // loads of the slot done and stores of the message visible, then both
            // hand-offs
            release_stores(local);
            __syncthreads();
            if (threadIdx.x == 0) {
                const bool drop = (a.inject & RR_INJECT_DROP_ARRIVAL) && injected && k == 0;
                if (has_send && !drop)
                    sig_add(&a.ready[(uint64_t)(lane * R + succ) * kSignalStride], 1);
                if (has_in) sig_add(&a.credit[(uint64_t)(lane * R + pred) * kSignalStride], 1);
            }
        }
    }
    if (synced && threadIdx.x == 0) {
        a.ready_shadow[my_slot] = ready_shadow;
        // every message this rank sends (K of them) is consumed and credited
        a.credit_shadow[my_slot] = credit_base + (uint64_t)K;
    }
    }  // rounds
}

template <int DT, int OP, int BLOCK>
__global__ void __launch_bounds__(BLOCK) staged_kernel(const StagedArgs a) {
    staged_body<DT, OP, BLOCK>(a, launch_generation(a.launch));
    leave_launch(a.launch);
}

// ---------------------------------------------------------------- AlltoAll
//
// The pure AlltoAll of the 2kiu.com article on NCCL GIN (section "a pure GIN
// AlltoAll kernel"): every rank puts block q of its send buffer into rank q's
// receive buffer at block position (its own rank), each put followed by one
// increment of the receiver's counting signal, and one receiving workgroup per
// rank waits until all the arrivals it expects have landed.  Workgroup (rank r,
// part p) copies part p of its R blocks, releases its stores at agent scope,
// then adds 1 to each receiver's signal; so a receiver expects R * parts
// arrivals per call (R with one part).  The waiter advances a persisted shadow
// (the article's per-signal shadows) instead of reading the signal at entry,
// which is why no entry barrier is needed here: there is no base value to race
// with.  Loads and stores are both non-temporal: each byte crosses once and the
// call never reads a receive buffer.  The stores are made at device scope
// (written through the L2, as an agent-scope store is on this chip), so a
// workgroup's puts are visible on every XCD once they are acknowledged, and the
// arrival needs no L2 write-back before it (which cost 4% at 8 ranks x 64 MiB).
struct A2AArgs {
    const void* send[kMaxDevices];
    void* recv[kMaxDevices];
    uint64_t count;     // elements per block
    uint64_t part_len;  // elements per part (a vector multiple)
    uint64_t* sig;      // one counting signal per receiver
    uint64_t* shadow;
    ErrorRecord* err;
    uint64_t timeout_ticks;
    int32_t R;
    int32_t parts;
    int32_t aligned;
    uint32_t inject;
};

template <int ES, int BLOCK>
__global__ void __launch_bounds__(BLOCK) alltoall_kernel(const A2AArgs a) {
    constexpr int V = 16 / ES;
    constexpr int U = kA2AUnroll;
    const int R = a.R;
    const int r = (int)blockIdx.x / a.parts;
    const int part = (int)blockIdx.x - r * a.parts;
    __shared__ int s_stop;
    if (threadIdx.x == 0) s_stop = sig_read(&a.err->flag) != 0;  // sticky failure
    __syncthreads();
    if (s_stop) return;
    const uint64_t lo = (uint64_t)part * a.part_len;
    const uint64_t hi = umin(lo + a.part_len, a.count);
    for (int i = 0; i < R && lo < hi; ++i) {
        const int q = (r + 1 + i) % R;  // start at the successor: spread the receivers
        const char* src = (const char*)a.send[r] + ((uint64_t)q * a.count + lo) * ES;
        char* dst = (char*)a.recv[q] + ((uint64_t)r * a.count + lo) * ES;
        const uint64_t n = hi - lo;
        // stores carry device scope (written through the L2) and the
        // non-temporal hint, through buffer descriptors of at most 1 GiB
        constexpr uint64_t kPieceElems = kPieceBytes / ES;
        for (uint64_t p0 = 0; p0 < n; p0 += kPieceElems) {
            const uint64_t m = umin(kPieceElems, n - p0);
            const char* sp = src + p0 * ES;
            const __amdgpu_buffer_rsrc_t out = incoming(dst + p0 * ES, m * ES);
            uint64_t done = 0;
            if (a.aligned) {
                const u32x4* __restrict__ s4 = (const u32x4*)sp;
                const uint32_t nv = (uint32_t)(m / V);
                uint32_t v = threadIdx.x;
                for (; v + (U - 1) * BLOCK < nv; v += U * BLOCK) {
                    u32x4 x[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(&s4[v + u * BLOCK]);
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        __builtin_amdgcn_raw_buffer_store_b128(x[u], out, (int)((v + u * BLOCK) * 16u),
                                                               0, kAuxStoreOut);
                }
                for (; v < nv; v += BLOCK)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_nontemporal_load(&s4[v]), out,
                                                           (int)(v * 16u), 0, kAuxStoreOut);
                done = (uint64_t)nv * V;
            }
            for (uint64_t t = done + threadIdx.x; t < m; t += BLOCK) {
                if constexpr (ES == 2)
                    __builtin_amdgcn_raw_buffer_store_b16(((const uint16_t*)sp)[t], out,
                                                          (int)(t * 2), 0, kAuxStoreOut);
                else
                    __builtin_amdgcn_raw_buffer_store_b32(((const uint32_t*)sp)[t], out,
                                                          (int)(t * 4), 0, kAuxStoreOut);
            }
        }
    }
    // the puts have landed before the receivers are told: every store above was
    // made at device scope, so once they are acknowledged they are visible on
    // every XCD, and no L2 write-back is needed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const bool drop = (a.inject & RR_INJECT_DROP_ARRIVAL) && r == 0 && part == 0;
    if (!drop && (int)threadIdx.x < R) sig_add(&a.sig[(uint64_t)threadIdx.x * kSignalStride], 1);
    if (part == 0 && threadIdx.x == 0) {  // the receiving workgroup of rank r
        uint64_t target = a.shadow[r] + (uint64_t)R * a.parts;
        if ((a.inject & RR_INJECT_EXTRA_EXPECTED) && r == 0) target += 1;
        const WaitResult res = sig_wait(&a.sig[(uint64_t)r * kSignalStride], target, a.err,
                                        a.timeout_ticks);
        if (res.status == WAIT_TIMEOUT) record_timeout(a.err, 0, r, 0, target, res.observed);
        if (res.status == WAIT_OK) a.shadow[r] = target;
    }
}

// ---------------------------------------------------------- barrier only --

struct BarrierArgs {
    uint64_t* sig;       // counting signals, one per (context, waiter)
    uint64_t* shadow;
    uint64_t* pp_sig;    // per-peer slots: a row of pp_row words per (context, waiter)
    uint64_t* pp_shadow;
    uint64_t* early;     // per (context, waiter): steps passed before every peer arrived
    uint64_t* xcc_table;
    ErrorRecord* err;
    uint64_t timeout_ticks;
    uint64_t expected;   // arrivals per step (counting) or per slot and step (per peer)
    int32_t R;           // waiters per context taking part
    int32_t stride;      // waiters per context in the object's layout
    int32_t pp_row;      // words per per-peer row
    int32_t nsteps;
    int32_t mode;        // SYNC_P2P, SYNC_BARRIER or SYNC_PER_PEER
    int32_t nctx;        // contexts taking part (columns; the grid is padded to 8)
    LaunchTag launch;
    uint64_t* stamps;    // optional: wall clock per (context, waiter): start, then each step
    uint32_t inject;
    int32_t audit;       // counting mode: also keep per-peer witnesses and count early passes
    int32_t pad;
};

struct PeerWait {
    int status;
    int lane;  // first unsatisfied lane on a timeout
    uint64_t expected, observed;
};

// Per-peer wait, for the whole wave: each active lane watches one slot until it
// reaches that lane's target; the wave leaves when every lane is satisfied.
// Every decision that ends the loop is wave-uniform.
__device__ PeerWait peer_wait(const uint64_t* slot, bool active, uint64_t target,
                              const ErrorRecord* err, uint64_t timeout_ticks) {
    uint64_t v = active ? sig_read(slot) : target;
    bool ok = !active || rolling_le(target, v);
    if (__all(ok)) return {WAIT_OK, -1, 0, 0};
    const uint64_t start = wall_clock64();
    uint32_t spins = 0;
    for (;;) {
        __builtin_amdgcn_s_sleep(1);
        if (!ok) {
            v = sig_read(slot);
            ok = rolling_le(target, v);
        }
        if (__all(ok)) return {WAIT_OK, -1, 0, 0};
        if ((++spins & 31u) == 0u) {
            const uint32_t stop =
                __builtin_amdgcn_readfirstlane((uint32_t)(sig_read(&err->flag) != 0));
            if (stop) return {WAIT_ABORT, -1, 0, 0};
            if (wall_clock64() - start > timeout_ticks) {
                const uint64_t bad = __ballot(!ok);
                const int lane = (int)__builtin_ctzll(bad);
                const uint64_t e = ((uint64_t)(uint32_t)__shfl((int)(target >> 32), lane) << 32) |
                                   (uint32_t)__shfl((int)(uint32_t)target, lane);
                const uint64_t o = ((uint64_t)(uint32_t)__shfl((int)(v >> 32), lane) << 32) |
                                   (uint32_t)__shfl((int)(uint32_t)v, lane);
                return {WAIT_TIMEOUT, lane, e, o};
            }
        }
    }
}

// One 64-lane workgroup (one wave) per (context, waiter), laid out like the ring
// kernel's columns so a context's waiters share an XCD.  Each step: release,
// arrive, advance the shadow, wait, acquire -- the same hand-off the ring kernel
// performs between hops, without the payload.  Lane i < R-1 serves the peer
// q = r+1+i (mod R): it arrives at q, and in per-peer mode it also watches
// q's slot in this waiter's row.
//
// Arrivals per step:
//   P2P       one add to the successor's counting signal
//   BARRIER   one add to each other waiter's counting signal; the waiter
//             expects R-1 on its own (the DeepEP pull request's counting barrier)
//   PER_PEER  one add to this waiter's slot in each other waiter's row; the
//             waiter expects every slot of its row to advance (the per-peer
//             layout the pull request replaced)
__device__ __forceinline__ void barrier_body(const BarrierArgs& a, const uint32_t generation) {
    const Place pl = place_of(blockIdx.x, a.R, true);
    const int r = pl.rank, ctx = pl.col;
    if (ctx >= a.nctx || a.nsteps <= 0) return;
    const int slot = ctx * a.stride + r;
    const uint32_t my_xcc = xcc_id() & 0xFu;
    __shared__ int s_stop;
    uint64_t shadow = 0;
    if (threadIdx.x == 0) {
        s_stop = sig_read(&a.err->flag) != 0;
        shadow = a.shadow[slot];
        publish_xcc(a.xcc_table, generation, my_xcc);
    }
    __syncthreads();
    if (s_stop) return;
    const int v = column_on_one_xcd(a.xcc_table, generation, a.R, ctx, true, my_xcc, a.err,
                                    a.timeout_ticks);
    if (v < 0) {
        if (threadIdx.x == 0) record_timeout(a.err, ctx, r, 0, generation, 0);
        return;
    }
    const bool local = v == 1;
    const bool injected = r == 0 && ctx == 0;
    const int lane = (int)threadIdx.x;
    const bool peer_lane = lane < a.R - 1;
    const int q = wrap(r + 1 + lane, a.R);
    const bool per_peer = a.mode == SYNC_PER_PEER;
    const bool audit = a.audit && a.mode == SYNC_BARRIER;
    const bool use_pp = per_peer || audit;
    // my slot in q's row (where I arrive) and q's slot in my row (what I watch)
    uint64_t* const out_pp = a.pp_sig + (uint64_t)(ctx * a.stride + q) * a.pp_row + r;
    uint64_t* const in_pp = a.pp_sig + (uint64_t)slot * a.pp_row + q;
    uint64_t* const in_pp_shadow = a.pp_shadow + (uint64_t)slot * a.pp_row + q;
    uint64_t pp_shadow = use_pp && peer_lane ? *in_pp_shadow : 0;
    uint64_t early = 0;
    // RR_INJECT_DEFER_ARRIVAL: waiter 0 of context 0 holds back its step-1 and
    // step-2 arrivals at waiter 1 until it has passed step 2 (with one step,
    // until the end).  Its step-2 arrival must be held too: otherwise it stands
    // in for its own late step-1 arrival, which both layouts allow.
    const bool defer = (a.inject & RR_INJECT_DEFER_ARRIVAL) && injected && peer_lane && q == 1;
    // optional timestamps: the constant-rate wall clock before the first step and
    // when each step's wait is over (lane 0 of the waiter's wave)
    uint64_t* const stamps =
        a.stamps ? a.stamps + (uint64_t)(ctx * a.R + r) * (uint64_t)(a.nsteps + 1) : nullptr;
    if (stamps && lane == 0) stamps[0] = wall_clock64();

    auto arrive = [&]() {
        if (per_peer) {
            sig_add(out_pp, 1);
            return;
        }
        if (audit) {
            // the witness is visible before the counting arrival it stands for
            sig_add(out_pp, 1);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        }
        sig_add(&a.sig[(uint64_t)(ctx * a.stride + q) * kSignalStride], 1);
    };

    for (int step = 1; step <= a.nsteps; ++step) {
        release_stores(local);
        const bool drop = (a.inject & RR_INJECT_DROP_ARRIVAL) && injected && step == 1;
        if (!drop) {
            if (a.mode == SYNC_P2P) {
                if (lane == 0) sig_add(&a.sig[(uint64_t)(ctx * a.stride + q) * kSignalStride], 1);
            } else if (peer_lane && !(defer && step <= 2)) {
                arrive();
            }
        }
        if (per_peer) {
            uint64_t target = pp_shadow + a.expected;
            if ((a.inject & RR_INJECT_EXTRA_EXPECTED) && injected && step == 1) target += 1;
            const PeerWait res = peer_wait(in_pp, peer_lane, target, a.err, a.timeout_ticks);
            if (res.status == WAIT_TIMEOUT && lane == 0)
                record_timeout(a.err, ctx, r, step, res.expected, res.observed,
                               wrap(r + 1 + res.lane, a.R));
            if (res.status != WAIT_OK) return;
            pp_shadow = target;
            if (lane == 0) acquire_stores(local);
            __syncthreads();
            if (stamps && lane == 0) stamps[step] = wall_clock64();
        } else {
            if (lane == 0) {
                uint64_t target = shadow + a.expected;
                if ((a.inject & RR_INJECT_EXTRA_EXPECTED) && injected && step == 1) target += 1;
                const WaitResult res = sig_wait(&a.sig[(uint64_t)slot * kSignalStride], target,
                                                a.err, a.timeout_ticks);
                if (res.status == WAIT_TIMEOUT)
                    record_timeout(a.err, ctx, r, step, target, res.observed);
                shadow = target;
                s_stop = res.status != WAIT_OK;
                acquire_stores(local);
            }
            __syncthreads();
            if (s_stop) return;
            if (stamps && lane == 0) stamps[step] = wall_clock64();
            if (audit) {
                bool missing = false;
                if (peer_lane) {
                    missing = !rolling_le(pp_shadow + 1, sig_read(in_pp));
                    pp_shadow += 1;
                }
                if (__any(missing)) early += 1;
            }
        }
        if (defer && step == 2) {
            arrive();
            arrive();
        }
    }
    if (defer && a.nsteps == 1) arrive();
    if (lane == 0) {
        if (!per_peer) a.shadow[slot] = shadow;
        if (audit) a.early[slot] += early;
    }
    if (use_pp && peer_lane) *in_pp_shadow = pp_shadow;
}

__global__ void __launch_bounds__(64) barrier_kernel(const BarrierArgs a) {
    barrier_body(a, launch_generation(a.launch));
    leave_launch(a.launch);
}

// ------------------------------------------------------ support kernels --

__global__ void __launch_bounds__(256) fill_u64_kernel(uint64_t* p, uint64_t n, uint64_t value,
                                                       uint64_t stride) {
    for (uint64_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += (uint64_t)gridDim.x * 256ull)
        p[i * stride] = value;
}

// Streaming copy: the bandwidth reference for the ring kernels.  Each
// workgroup copies one contiguous span (DRAM pages stay open longer than with a
// grid-wide stride); nontemporal hints, as the data are touched once.  1024
// threads x 8 vectors in flight, 2 workgroups per CU: 6.06-6.08 TB/s on MI355X,
// the best of a probe over span layouts, hints, grids of 256-4096, 256-1024
// threads and 4-16 vectors per thread (512 threads x 8, 4 per CU: 5.82-5.91;
// 256-thread workgroups: 5.6 at any grid size).
__global__ void __launch_bounds__(kCopyBlock) copy_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, uint64_t nvec,
                                                          const uint8_t* __restrict__ src_tail,
                                                          uint8_t* __restrict__ dst_tail,
                                                          uint32_t ntail) {
    constexpr int U = 8;
    constexpr int B = kCopyBlock;
    const uint64_t per = (nvec + gridDim.x - 1) / gridDim.x;
    const uint64_t lo = (uint64_t)blockIdx.x * per;
    const uint64_t hi = lo + per < nvec ? lo + per : nvec;
    uint64_t i = lo + threadIdx.x;
    for (; i + (U - 1) * B < hi; i += U * B) {
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(&src[i + u * B]);
#pragma unroll
        for (int u = 0; u < U; ++u) __builtin_nontemporal_store(x[u], &dst[i + u * B]);
    }
    for (; i < hi; i += B) dst[i] = src[i];
    if (blockIdx.x == 0 && threadIdx.x < ntail) dst_tail[threadIdx.x] = src_tail[threadIdx.x];
}

// ------------------------------------------------------------- host side --

struct DeviceState {
    bool ready = false;
    int cus = 0;
    int wall_khz = 0;
    uint64_t* mem = nullptr;
    uint64_t* sig = nullptr;
    uint64_t* shadow = nullptr;
    uint64_t* xcc_table = nullptr;
    ErrorRecord* err = nullptr;
    uint64_t* credit = nullptr;         // staged loop: slot-free signals, one per cache line
    uint64_t* credit_shadow = nullptr;
    char* fifo = nullptr;               // staged loop: receive buffers, grown on demand
    size_t fifo_bytes = 0;
    uint64_t* launch_gen = nullptr;     // per-launch tag of the XCD table (starts at 1)
    uint64_t* launch_exits = nullptr;   // workgroups of the running launch that have left
};

std::mutex g_mu;
DeviceState g_dev[kMaxDevices];

struct Plan {
    int long_nap;
    int stream_in;
    int fuse;
    int sync;
    int team;
    int rounds;
    int depth;
    int cols;
    int block;
    int grid;
    int launches;
    int xcd_map;
    int coop;
    int resident_max;
    uint64_t chunk_len, slice_len, sub_len, hbm_bytes;
    int g_first, g_last;
};

static inline uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }
static inline uint64_t round_up(uint64_t a, uint64_t b) { return ceil_div(a, b) * b; }

static size_t elem_bytes(int dt) { return dt == RR_BF16 || dt == RR_FP16 ? 2 : 4; }

static bool hip_ok(hipError_t e) { return e == hipSuccess; }

static rr_status_t ensure_device(DeviceState** out) {
    int dev = 0;
    if (!hip_ok(hipGetDevice(&dev))) return RR_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return RR_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState& d = g_dev[dev];
    if (!d.ready) {
        if (!hip_ok(hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev)))
            return RR_ERR_HIP;
        if (!hip_ok(hipDeviceGetAttribute(&d.wall_khz, hipDeviceAttributeWallClockRate, dev)) ||
            d.wall_khz <= 0)
            d.wall_khz = 100000;  // the gfx9 constant-rate clock runs at 100 MHz
        // signals (one per cache line), shadows, the XCC table, the error record,
        // the staged loop's credit signals and their shadows, then the launch tag
        // and the exit count (a cache line each)
        const size_t words = 2 * ((size_t)kSlots * kSignalStride + (size_t)kSlots) +
                             (size_t)kSlots + 16 + 2 * kSignalStride;
        void* p = nullptr;
        if (!hip_ok(hipMalloc(&p, words * sizeof(uint64_t)))) return RR_ERR_NOMEM;
        if (!hip_ok(hipMemset(p, 0, words * sizeof(uint64_t)))) {
            (void)hipFree(p);
            return RR_ERR_HIP;
        }
        d.mem = (uint64_t*)p;
        d.sig = d.mem;
        d.shadow = d.mem + (size_t)kSlots * kSignalStride;
        d.xcc_table = d.shadow + kSlots;
        d.err = (ErrorRecord*)(d.xcc_table + kSlots);
        d.credit = d.xcc_table + kSlots + 16;
        d.credit_shadow = d.credit + (size_t)kSlots * kSignalStride;
        d.launch_gen = d.credit_shadow + kSlots;
        d.launch_exits = d.launch_gen + kSignalStride;
        const uint64_t first_tag = 1;
        if (!hip_ok(hipMemcpy(d.launch_gen, &first_tag, sizeof first_tag,
                              hipMemcpyHostToDevice))) {
            (void)hipFree(p);
            return RR_ERR_HIP;
        }
        d.ready = true;
    }
    *out = &d;
    return RR_OK;
}

static uint64_t timeout_ticks(const DeviceState* d, const rr_options_t* opt) {
    const uint64_t ns = opt && opt->timeout_ns ? opt->timeout_ns : kDefaultTimeoutNs;
    return ns / 1000ull * (uint64_t)d->wall_khz / 1000ull + 1;
}

typedef void (*RingKernel)(RingArgs);

template <int DT, int OP>
static RingKernel ring_kernel_for_block(int block) {
    switch (block) {
        case 128: return ring_kernel<DT, OP, 128>;
        case 256: return ring_kernel<DT, OP, 256>;
        case 512: return ring_kernel<DT, OP, 512>;
        case 1024: return ring_kernel<DT, OP, 1024>;
        default: return nullptr;
    }
}

template <int DT>
static RingKernel ring_kernel_for_op(int op, int block) {
    switch (op) {
        case RR_SUM: return ring_kernel_for_block<DT, OP_SUM>(block);
        case RR_MAX: return ring_kernel_for_block<DT, OP_MAX>(block);
        case RR_MIN: return ring_kernel_for_block<DT, OP_MIN>(block);
        case RR_PROD: return ring_kernel_for_block<DT, OP_PROD>(block);
        default: return nullptr;
    }
}

static RingKernel pick_ring_kernel(int dt, int op, int block) {
    switch (dt) {
        case RR_INT32: return ring_kernel_for_op<DT_I32>(op, block);
        case RR_FP32: return ring_kernel_for_op<DT_F32>(op, block);
        case RR_BF16: return ring_kernel_for_op<DT_BF16>(op, block);
        case RR_FP16: return ring_kernel_for_op<DT_F16>(op, block);
        default: return nullptr;
    }
}

typedef void (*StagedKernel)(StagedArgs);

template <int DT>
static StagedKernel staged_kernel_for_op(int op) {
    switch (op) {
        case RR_SUM: return staged_kernel<DT, OP_SUM, kStagedBlock>;
        case RR_MAX: return staged_kernel<DT, OP_MAX, kStagedBlock>;
        case RR_MIN: return staged_kernel<DT, OP_MIN, kStagedBlock>;
        case RR_PROD: return staged_kernel<DT, OP_PROD, kStagedBlock>;
        default: return nullptr;
    }
}

static StagedKernel pick_staged_kernel(int dt, int op) {
    switch (dt) {
        case RR_INT32: return staged_kernel_for_op<DT_I32>(op);
        case RR_FP32: return staged_kernel_for_op<DT_F32>(op);
        case RR_BF16: return staged_kernel_for_op<DT_BF16>(op);
        case RR_FP16: return staged_kernel_for_op<DT_F16>(op);
        default: return nullptr;
    }
}

static bool valid_dtype(int dt) {
    return dt == RR_INT32 || dt == RR_FP32 || dt == RR_BF16 || dt == RR_FP16;
}
static bool valid_op(int op) { return op == RR_SUM || op == RR_MAX || op == RR_MIN || op == RR_PROD; }

// Argument checks that need no device.
// Option and size limits of each call family (phase numbering of
// rr_plan_query), shared by the calls and the plan query so that both reject
// the same arguments.
static rr_status_t check_shape(int R, uint64_t count, int phase, const rr_options_t* opt) {
    if (R < 1 || R > RR_MAX_RANKS) return RR_ERR_INVALID;
    const uint64_t kMaxElems = (uint64_t)1 << 40;
    if (phase <= 2) {
        if (count > kMaxElems) return RR_ERR_INVALID;
    } else if (count > kMaxElems || (uint64_t)R * count > kMaxElems) {
        return RR_ERR_INVALID;
    }
    if (!opt) return RR_OK;
    const int max_sync = phase == 6 ? RR_SYNC_P2P : RR_SYNC_LAUNCH;
    if (opt->sync < RR_SYNC_AUTO || opt->sync > max_sync) return RR_ERR_INVALID;
    if (opt->team < 0 || opt->team > (phase == 6 ? 65536 : 4096)) return RR_ERR_INVALID;
    if (phase == 6) return RR_OK;
    if (opt->rounds < 0 || opt->rounds > 4096) return RR_ERR_INVALID;
    if (phase <= 2 && (opt->depth < 0 || opt->depth > kMaxDepth)) return RR_ERR_INVALID;
    if (opt->block != 0 && opt->block != 128 && opt->block != 256 && opt->block != 512 &&
        opt->block != 1024)
        return RR_ERR_INVALID;
    return RR_OK;
}

static rr_status_t check_args(void* const* bufs, int R, size_t count, int dt, int op, int nslices,
                              const rr_options_t* opt) {
    if (R < 1 || R > RR_MAX_RANKS) return RR_ERR_INVALID;
    if (nslices < 1 || nslices > RR_MAX_SLICES) return RR_ERR_INVALID;
    if (!valid_dtype(dt) || !valid_op(op)) return RR_ERR_INVALID;
    const rr_status_t st = check_shape(R, count, 0, opt);
    if (st != RR_OK) return st;
    if (!bufs) return RR_ERR_INVALID;
    if (R == 1 || count == 0) return RR_OK;
    const size_t bytes = count * elem_bytes(dt);
    std::vector<uintptr_t> p((size_t)R);
    for (int r = 0; r < R; ++r) {
        if (!bufs[r]) return RR_ERR_INVALID;
        p[(size_t)r] = (uintptr_t)bufs[r];
        if (p[(size_t)r] % 16 != 0) return RR_ERR_INVALID;
    }
    std::sort(p.begin(), p.end());
    for (int r = 0; r + 1 < R; ++r)
        if (p[(size_t)r] + bytes > p[(size_t)r + 1]) return RR_ERR_INVALID;
    return RR_OK;
}

// Every buffer must lie inside one allocation of the current device, so that no
// kernel can touch memory outside what the caller handed over.
static rr_status_t check_extents(void* const* bufs, int R, size_t bytes) {
    int dev = 0;
    if (!hip_ok(hipGetDevice(&dev))) return RR_ERR_HIP;
    for (int r = 0; r < R; ++r) {
        hipPointerAttribute_t attr;
        if (!hip_ok(hipPointerGetAttributes(&attr, bufs[r]))) {
            (void)hipGetLastError();
            return RR_ERR_INVALID;
        }
        if (attr.type != hipMemoryTypeDevice || attr.device != dev) return RR_ERR_INVALID;
        hipDeviceptr_t base = nullptr;
        size_t size = 0;
        if (!hip_ok(hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)bufs[r]))) {
            (void)hipGetLastError();
            return RR_ERR_INVALID;
        }
        if ((uintptr_t)bufs[r] + bytes > (uintptr_t)base + size) return RR_ERR_INVALID;
    }
    return RR_OK;
}

static int resident_limit(const DeviceState* d, const void* kernel, int block) {
    int per_cu = 0;
    if (!hip_ok(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0))) {
        (void)hipGetLastError();
        return 0;
    }
    return per_cu * d->cus;
}

// phase: 0 AllReduce, 1 ReduceScatter, 2 AllGather.
static rr_status_t make_plan(const DeviceState* d, int R, size_t count, int dt, int op,
                             int nslices, int phase, const rr_options_t* opt, Plan* p) {
    const uint64_t V = 16 / elem_bytes(dt);
    const bool fixed_block = opt && opt->block;
    int block = fixed_block ? opt->block : kAutoBlock;
    const int requested = opt ? opt->sync : RR_SYNC_AUTO;
    const uint32_t flags = opt ? opt->flags : 0;
    if ((flags & RR_FLAG_STREAM_LOADS) && (flags & RR_FLAG_CACHED_LOADS)) return RR_ERR_INVALID;
    p->chunk_len = round_up(ceil_div(count, (uint64_t)R), V);
    p->slice_len = round_up(ceil_div(p->chunk_len, (uint64_t)nslices), V);
    if (phase == 0) {
        p->g_first = 1;
        p->g_last = 2 * (R - 1);
    } else if (phase == 1) {
        p->g_first = 1;
        p->g_last = R - 1;
    } else {
        p->g_first = R;
        p->g_last = 2 * (R - 1);
    }
    const uint64_t nbytes = (uint64_t)count * elem_bytes(dt);
    const uint64_t rs = phase != 2 ? 3ull * (uint64_t)(R - 1) * nbytes : 0;
    const uint64_t ag = phase != 1 ? 2ull * (uint64_t)(R - 1) * nbytes : 0;
    // fusion applies to a whole AllReduce only; it saves the first AllGather
    // hop's load: one chunk per rank, N bytes in all
    p->fuse = phase == 0 && R > 1 && (flags & RR_FLAG_FUSED_BOUNDARY) ? 1 : 0;
    p->hbm_bytes = R > 1 ? rs + ag - (p->fuse ? nbytes : 0) : 0;

    // Workgroups per rank (cols): about 16 waves per CU, two 512-thread
    // workgroups.  Each interleaves `depth` lanes and runs `rounds` groups of
    // them one after another; rounds bound one hop of the lanes in flight
    // (3 N / rounds bytes over all ranks), so that a partial is still cached
    // when the next hop reads it.
    const int target_cols = std::max(1, d->cus * 16 * 64 / block / R);
    const bool fixed_depth = opt && opt->depth > 0;
    const bool fixed_rounds = opt && opt->rounds > 0;
    const bool barrier = requested == RR_SYNC_BARRIER;
    const uint64_t hop_bytes = 3ull * (uint64_t)count * elem_bytes(dt);
    const bool wide = !barrier && R >= kLongRingRanks && hop_bytes >= kWideHopBytes;
    int depth = fixed_depth ? opt->depth
                            : (barrier ? kAutoDepthBarrier : wide ? kAutoDepthWide : kAutoDepthP2P);
    int rounds;
    if (fixed_rounds) {
        rounds = opt->rounds;
    } else {
        const uint64_t per_round =
            barrier ? std::min(kBarrierRoundMax,
                               std::max(kBarrierRoundMin, (uint64_t)R * kBarrierRoundPerRank))
            : wide  ? kWideRoundBytes
                    : std::max<uint64_t>(kRoundBytesMin, (uint64_t)R * kRoundBytesPerRank);
        uint64_t k = 1;  // a power of two: lanes split evenly over the XCDs
        while (k * per_round < hop_bytes) k *= 2;
        rounds = (int)k;
    }
    int team;
    const uint64_t slice_vecs = p->slice_len / V;
    const uint64_t min_vecs = (uint64_t)block * 4;  // one unrolled pass per hop
    const uint64_t by_size = std::max<uint64_t>(1, slice_vecs / min_vecs);
    auto auto_team = [&](int dd) {
        const uint64_t wanted = ceil_div((uint64_t)target_cols * dd * rounds, nslices);
        return (int)std::max<uint64_t>(1, std::min<uint64_t>(by_size, wanted));
    };
    if (opt && opt->team > 0) {
        team = opt->team;
    } else {
        team = auto_team(depth);
        // Interleaving pays only when the buffer can fill at least half the
        // columns wanted; a smaller one would just serialise two lanes'
        // hand-offs in one workgroup (R=16: 4 MiB per rank and below).
        if (!fixed_depth && depth > 1 &&
            2 * (uint64_t)nslices * team / ((uint64_t)depth * rounds) < (uint64_t)target_cols) {
            depth = 1;
            team = auto_team(1);
        }
    }
    // every lane needs R signals in the workspace
    const int max_team = std::max(1, kSlots / (R * nslices));
    if (team > max_team) {
        if (opt && opt->team > 0) return RR_ERR_UNSUPPORTED;
        team = max_team;
    }
    const int lanes = nslices * team;
    // depth * rounds must divide the lanes; automatic choices shrink to fit
    auto fits = [&](int dd, int kk) { return dd * kk <= lanes && lanes % (dd * kk) == 0; };
    if (!fits(depth, rounds)) {
        if (fixed_depth && fixed_rounds) return RR_ERR_UNSUPPORTED;
        int best_d = 1, best_k = 1;
        for (int dd = depth; dd >= 1; --dd) {
            if (fixed_depth && dd != depth) continue;
            for (int kk = rounds; kk >= 1; --kk) {
                if (fixed_rounds && kk != rounds) continue;
                if (fits(dd, kk) && dd * kk > best_d * best_k) {
                    best_d = dd;
                    best_k = kk;
                }
            }
        }
        if (!fits(best_d, best_k) || (fixed_depth && best_d != depth) ||
            (fixed_rounds && best_k != rounds))
            return RR_ERR_UNSUPPORTED;
        depth = best_d;
        rounds = best_k;
    }
    p->team = team;
    p->depth = depth;
    p->rounds = rounds;
    p->cols = lanes / (depth * rounds);
    p->sub_len = round_up(ceil_div(p->slice_len, (uint64_t)team), V);
    if (!fixed_block) {
        const uint64_t piece = p->sub_len * elem_bytes(dt);
        if (piece <= kTinyPieceBytes)
            block = kSmallBlock;
        else if (piece > kMidPieceLo && piece <= kMidPieceHi)
            block = kMidBlock;
        else if (R >= kLongRingRanks && (uint64_t)R * nbytes > kInfinityCacheBytes &&
                 piece <= kLongRingPieceBytes)
            block = kSmallBlock;
    }
    p->block = block;
    const void* kernel = (const void*)pick_ring_kernel(dt, op, block);
    p->resident_max = resident_limit(d, kernel, block);
    // Columns on the XCD map are padded to a multiple of 8 (idle columns exit).
    p->xcd_map = (flags & RR_FLAG_NO_XCD_MAP) ? 0 : 1;
    const uint64_t cols_launched = p->xcd_map ? round_up((uint64_t)p->cols, 8) : p->cols;
    if ((uint64_t)R * cols_launched > (1ull << 30)) return RR_ERR_INVALID;
    p->grid = (int)(R * cols_launched);

    const bool multi_hop = p->g_last > p->g_first;
    int sync = requested;
    if (sync == RR_SYNC_AUTO) sync = multi_hop && p->grid <= p->resident_max ? RR_SYNC_P2P : RR_SYNC_LAUNCH;
    if ((sync == RR_SYNC_P2P || sync == RR_SYNC_BARRIER) && multi_hop &&
        (p->grid > p->resident_max || p->grid > kSlots))  // the XCC table has kSlots entries
        return RR_ERR_UNSUPPORTED;
    if (!multi_hop && sync != RR_SYNC_LAUNCH) sync = RR_SYNC_LAUNCH;  // one hop needs no hand-off
    p->sync = sync;
    p->launches = sync == RR_SYNC_LAUNCH ? p->g_last - p->g_first + 1 : 1;
    p->coop = sync != RR_SYNC_LAUNCH && (flags & RR_FLAG_COOPERATIVE) ? 1 : 0;
    // barrier waits poll slowly once one hop moves at least kLongNapBytes over
    // all ranks (about 10 us of traffic, so a later wake-up of up to ~2 us is
    // hidden; smaller buffers are latency-bound and keep the fast poll)
    p->long_nap = sync == RR_SYNC_BARRIER && 3ull * count * elem_bytes(dt) >= kLongNapBytes;
    p->stream_in = (flags & RR_FLAG_STREAM_LOADS) ||
                   (!(flags & RR_FLAG_CACHED_LOADS) && (uint64_t)R * nbytes > kInfinityCacheBytes);
    return RR_OK;
}

static rr_status_t run_ring(void* const* bufs, int R, size_t count, int dt, int op, int nslices,
                            int phase, const rr_options_t* opt, rr_stream_t stream) {
    rr_status_t st = check_args(bufs, R, count, dt, op, nslices, opt);
    if (st != RR_OK || R == 1 || count == 0) return st;
    DeviceState* d = nullptr;
    if ((st = ensure_device(&d)) != RR_OK) return st;
    if (!(opt && (opt->flags & RR_FLAG_NO_POINTER_CHECK)))
        if ((st = check_extents(bufs, R, count * elem_bytes(dt))) != RR_OK) return st;
    Plan p;
    if ((st = make_plan(d, R, count, dt, op, nslices, phase, opt, &p)) != RR_OK) return st;

    RingArgs a;
    memset(&a, 0, sizeof a);
    for (int r = 0; r < R; ++r) a.bufs[r] = bufs[r];
    a.count = count;
    a.chunk_len = p.chunk_len;
    a.slice_len = p.slice_len;
    a.sub_len = p.sub_len;
    a.sig = d->sig;
    a.shadow = d->shadow;
    a.xcc_table = d->xcc_table;
    a.err = d->err;
    a.timeout_ticks = timeout_ticks(d, opt);
    a.launch = {d->launch_gen, d->launch_exits};
    a.R = R;
    a.team = p.team;
    a.cols = p.cols;
    a.rounds = p.rounds;
    a.depth = p.depth;
    a.fuse = p.fuse;
    a.long_nap = p.long_nap;
    a.stream_in = p.stream_in;
    a.xcd_map = p.xcd_map;
    a.inject = opt ? opt->inject : 0;
    RingKernel k = pick_ring_kernel(dt, op, p.block);
    hipStream_t s = (hipStream_t)stream;
    if (p.sync == RR_SYNC_LAUNCH) {
        a.sync = SYNC_NONE;
        for (int g = p.g_first; g <= p.g_last; ++g) {
            a.g_first = a.g_last = g;
            hipLaunchKernelGGL(k, dim3(p.grid), dim3(p.block), 0, s, a);
        }
    } else {
        a.sync = p.sync == RR_SYNC_BARRIER ? SYNC_BARRIER : SYNC_P2P;
        a.g_first = p.g_first;
        a.g_last = p.g_last;
        void* args[] = {&a};
        if (p.coop) {
            if (!hip_ok(hipLaunchCooperativeKernel((const void*)k, dim3(p.grid), dim3(p.block), args,
                                                   0, s))) {
                (void)hipGetLastError();
                return RR_ERR_HIP;
            }
        } else {
            hipLaunchKernelGGL(k, dim3(p.grid), dim3(p.block), 0, s, a);
        }
    }
    if (!hip_ok(hipGetLastError())) return RR_ERR_HIP;
    return RR_OK;
}

// ------------------------------------------------------ the staged loop, host

static int staged_last_step(int R, int mode) { return mode == MODE_ALLREDUCE ? 2 * R - 2 : R - 1; }

// n: AllReduce elements per rank; ReduceScatter / AllGather elements per block.
static rr_status_t make_staged_plan(const DeviceState* d, int R, uint64_t n, int dt, int op,
                                    int nslices, int mode, const rr_options_t* opt, Plan* p) {
    const uint64_t es = elem_bytes(dt);
    const uint64_t V = 16 / es;
    const int requested = opt ? opt->sync : RR_SYNC_AUTO;
    const uint32_t flags = opt ? opt->flags : 0;
    if (opt && opt->block != 0 && opt->block != kStagedBlock) return RR_ERR_UNSUPPORTED;
    if (requested == RR_SYNC_BARRIER) return RR_ERR_UNSUPPORTED;  // credits pace the loop
    p->block = kStagedBlock;
    p->fuse = 0;
    p->stream_in = 0;
    p->chunk_len = mode == MODE_ALLREDUCE ? round_up(ceil_div(n, (uint64_t)R), V) : n;
    p->slice_len = round_up(ceil_div(p->chunk_len, (uint64_t)nslices), V);
    p->g_first = 0;
    p->g_last = staged_last_step(R, mode);
    p->hbm_bytes = R < 2 ? 0
                   : mode == MODE_ALLREDUCE ? (6ull * R - 4) * n * es
                                            : (3ull * R - 1) * (uint64_t)R * n * es;
    const void* kernel = (const void*)pick_staged_kernel(dt, mode == MODE_AG ? RR_SUM : op);
    if (!kernel) return RR_ERR_INVALID;
    p->resident_max = resident_limit(d, kernel, kStagedBlock);
    const int target_cols = std::max(1, d->cus * 16 * 64 / kStagedBlock / R);
    // rounds (a power of two): one step of the lanes in flight (reads and
    // writes of about three chunks per rank) within the step budget
    const uint64_t step_bytes = 3ull * (uint64_t)R * p->chunk_len * es;
    const uint64_t budget =
        mode == MODE_AG ? std::max<uint64_t>(kGatherRoundMin, kGatherRoundSpan / (uint64_t)R)
                        : kStagedRoundBytes;
    uint64_t k = 1;
    while (k * budget < step_bytes) k *= 2;
    int rounds = opt && opt->rounds > 0 ? opt->rounds : (int)k;
    int team;
    if (opt && opt->team > 0) {
        team = opt->team;
    } else {
        const uint64_t by_size = std::max<uint64_t>(1, p->slice_len / V / ((uint64_t)kStagedBlock * 4));
        const uint64_t wanted = ceil_div((uint64_t)target_cols * rounds, (uint64_t)nslices);
        team = (int)std::max<uint64_t>(1, std::min<uint64_t>(by_size, wanted));
    }
    const int max_team = std::max(1, kSlots / (R * nslices));
    if (team > max_team) {
        if (opt && opt->team > 0) return RR_ERR_UNSUPPORTED;
        team = max_team;
    }
    const int lanes = nslices * team;
    if (lanes % rounds != 0 || rounds > lanes) {  // rounds must divide the lanes
        if (opt && opt->rounds > 0) return RR_ERR_UNSUPPORTED;
        while (rounds > 1 && lanes % rounds != 0) --rounds;
    }
    p->team = team;
    p->depth = 1;
    p->rounds = rounds;
    p->cols = lanes / rounds;
    p->sub_len = round_up(ceil_div(p->slice_len, (uint64_t)team), V);
    p->xcd_map = (flags & RR_FLAG_NO_XCD_MAP) ? 0 : 1;
    const uint64_t cols_launched = p->xcd_map ? round_up((uint64_t)p->cols, 8) : p->cols;
    if ((uint64_t)R * cols_launched > (1ull << 30)) return RR_ERR_INVALID;
    p->grid = (int)(R * cols_launched);
    int sync = requested;
    if (sync == RR_SYNC_AUTO) sync = p->grid <= p->resident_max ? RR_SYNC_P2P : RR_SYNC_LAUNCH;
    if (sync == RR_SYNC_P2P && (p->grid > p->resident_max || p->grid > kSlots))
        return RR_ERR_UNSUPPORTED;
    p->sync = sync;
    p->launches = sync == RR_SYNC_LAUNCH ? p->g_last + 1 : 1;
    p->coop = 0;
    return RR_OK;
}

// Send and receive buffers: non-null, 16-byte aligned, pairwise disjoint,
// except that an AllReduce may receive in place (recv[r] == send[r]).
static rr_status_t check_staged_args(const void* const* send, void* const* recv, int R, uint64_t n,
                                     int dt, int op, int nslices, int mode, const rr_options_t* opt) {
    if (R < 1 || R > RR_MAX_RANKS || nslices < 1 || nslices > RR_MAX_SLICES) return RR_ERR_INVALID;
    if (!valid_dtype(dt) || !valid_op(op)) return RR_ERR_INVALID;
    const rr_status_t st = check_shape(R, n, 3 + mode, opt);
    if (st != RR_OK) return st;
    if (!send || !recv) return RR_ERR_INVALID;
    if (n == 0) return RR_OK;
    const uint64_t es = elem_bytes(dt);
    const uint64_t sbytes = (mode == MODE_RS ? (uint64_t)R : 1) * n * es;
    const uint64_t rbytes = (mode == MODE_AG ? (uint64_t)R : 1) * n * es;
    std::vector<std::pair<uintptr_t, uint64_t>> iv;
    for (int r = 0; r < R; ++r) {
        if (!send[r] || !recv[r]) return RR_ERR_INVALID;
        if ((uintptr_t)send[r] % 16 || (uintptr_t)recv[r] % 16) return RR_ERR_INVALID;
        iv.push_back({(uintptr_t)send[r], sbytes});
        const bool in_place = mode == MODE_ALLREDUCE && (const void*)recv[r] == send[r];
        if (!in_place) iv.push_back({(uintptr_t)recv[r], rbytes});
    }
    std::sort(iv.begin(), iv.end());
    for (size_t i = 0; i + 1 < iv.size(); ++i)
        if (iv[i].first + iv[i].second > iv[i + 1].first) return RR_ERR_INVALID;
    return RR_OK;
}

static rr_status_t ensure_fifo(DeviceState* d, size_t bytes) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (d->fifo_bytes >= bytes) return RR_OK;
    if (d->fifo) {
        if (!hip_ok(hipDeviceSynchronize())) return RR_ERR_HIP;
        (void)hipFree(d->fifo);
        d->fifo = nullptr;
        d->fifo_bytes = 0;
    }
    void* p = nullptr;
    if (!hip_ok(hipMalloc(&p, bytes))) return RR_ERR_NOMEM;
    d->fifo = (char*)p;
    d->fifo_bytes = bytes;
    return RR_OK;
}

static rr_status_t copy_bytes(void* dst, const void* src, uint64_t bytes, const DeviceState* d,
                              hipStream_t s) {
    const uint64_t nvec = bytes / 16;
    const uint32_t ntail = (uint32_t)(bytes % 16);
    const unsigned grid = (unsigned)std::max<uint64_t>(
        1, std::min<uint64_t>((uint64_t)d->cus * kCopyPerCU, ceil_div(nvec, 8 * kCopyBlock)));
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(kCopyBlock), 0, s, (const u32x4*)src, (u32x4*)dst,
                       nvec, (const uint8_t*)src + nvec * 16, (uint8_t*)dst + nvec * 16, ntail);
    return hip_ok(hipGetLastError()) ? RR_OK : RR_ERR_HIP;
}

static rr_status_t run_staged(const void* const* send, void* const* recv, int R, uint64_t n, int dt,
                              int op, int nslices, int mode, const rr_options_t* opt,
                              rr_stream_t stream) {
    rr_status_t st = check_staged_args(send, recv, R, n, dt, op, nslices, mode, opt);
    if (st != RR_OK || n == 0) return st;
    DeviceState* d = nullptr;
    if ((st = ensure_device(&d)) != RR_OK) return st;
    const uint64_t es = elem_bytes(dt);
    const uint64_t sbytes = (mode == MODE_RS ? (uint64_t)R : 1) * n * es;
    const uint64_t rbytes = (mode == MODE_AG ? (uint64_t)R : 1) * n * es;
    if (!(opt && (opt->flags & RR_FLAG_NO_POINTER_CHECK))) {
        if ((st = check_extents((void* const*)send, R, sbytes)) != RR_OK) return st;
        if ((st = check_extents(recv, R, rbytes)) != RR_OK) return st;
    }
    hipStream_t s = (hipStream_t)stream;
    if (R == 1) {  // nothing to exchange: the output is the input
        if ((const void*)recv[0] == send[0]) return RR_OK;
        return copy_bytes(recv[0], send[0], n * es, d, s);
    }
    Plan p;
    if ((st = make_staged_plan(d, R, n, dt, op, nslices, mode, opt, &p)) != RR_OK) return st;
    const uint64_t slot_len = round_up(p.chunk_len, 16 / es);
    if ((st = ensure_fifo(d, (size_t)R * kFifoSlots * slot_len * es)) != RR_OK) return st;

    StagedArgs a;
    memset(&a, 0, sizeof a);
    for (int r = 0; r < R; ++r) {
        a.send[r] = send[r];
        a.recv[r] = recv[r];
    }
    a.fifo = d->fifo;
    a.slot_len = slot_len;
    a.n = n;
    a.chunk_len = p.chunk_len;
    a.slice_len = p.slice_len;
    a.sub_len = p.sub_len;
    a.ready = d->sig;
    a.ready_shadow = d->shadow;
    a.credit = d->credit;
    a.credit_shadow = d->credit_shadow;
    a.xcc_table = d->xcc_table;
    a.err = d->err;
    a.timeout_ticks = timeout_ticks(d, opt);
    a.launch = {d->launch_gen, d->launch_exits};
    a.inject = opt ? opt->inject : 0;
    a.R = R;
    a.team = p.team;
    a.cols = p.cols;
    a.rounds = p.rounds;
    a.mode = mode;
    a.xcd_map = p.xcd_map;
    a.aligned = mode == MODE_ALLREDUCE || (n * es) % 16 == 0;
    StagedKernel k = pick_staged_kernel(dt, mode == MODE_AG ? RR_SUM : op);
    if (p.sync == RR_SYNC_LAUNCH) {
        for (int step = p.g_first; step <= p.g_last; ++step) {
            a.k_first = a.k_last = step;
            hipLaunchKernelGGL(k, dim3(p.grid), dim3(p.block), 0, s, a);
        }
    } else {
        a.k_first = p.g_first;
        a.k_last = p.g_last;
        hipLaunchKernelGGL(k, dim3(p.grid), dim3(p.block), 0, s, a);
    }
    return hip_ok(hipGetLastError()) ? RR_OK : RR_ERR_HIP;
}

// ------------------------------------------------------------- AlltoAll, host

static rr_status_t make_a2a_plan(const DeviceState* d, int R, uint64_t count, int dt,
                                 const rr_options_t* opt, Plan* p) {
    const uint64_t es = elem_bytes(dt);
    const uint64_t V = 16 / es;
    const void* kernel = es == 2 ? (const void*)alltoall_kernel<2, kA2ABlock>
                                 : (const void*)alltoall_kernel<4, kA2ABlock>;
    p->block = kA2ABlock;
    p->resident_max = resident_limit(d, kernel, kA2ABlock);
    // parts per block: about kA2AWavesPerCU waves per CU in all, every
    // workgroup resident (the receiving workgroups wait for the others)
    const uint64_t by_size = std::max<uint64_t>(1, count / V / ((uint64_t)kA2ABlock * kA2AUnroll));
    const uint64_t wanted = std::max<uint64_t>(
        1, std::min<uint64_t>((uint64_t)d->cus * kA2AWavesPerCU * 64 / kA2ABlock,
                              (uint64_t)p->resident_max) / (uint64_t)R);
    int parts = opt && opt->team > 0 ? opt->team
                                     : (int)std::max<uint64_t>(1, std::min<uint64_t>(by_size, wanted));
    p->team = parts;
    p->cols = parts;
    p->rounds = 1;
    p->depth = 1;
    p->fuse = 0;
    p->stream_in = 0;
    p->chunk_len = count;
    p->slice_len = count;
    p->sub_len = round_up(ceil_div(count, (uint64_t)parts), V);
    p->grid = R * parts;
    p->sync = RR_SYNC_P2P;
    p->launches = 1;
    p->xcd_map = 0;
    p->coop = 0;
    p->g_first = p->g_last = 0;
    p->hbm_bytes = 2ull * R * R * count * es;
    if (p->grid > p->resident_max) return RR_ERR_UNSUPPORTED;
    return RR_OK;
}

static rr_status_t run_alltoall(const void* const* send, void* const* recv, int R, uint64_t count,
                                int dt, const rr_options_t* opt, rr_stream_t stream) {
    if (R < 1 || R > RR_MAX_RANKS || !valid_dtype(dt)) return RR_ERR_INVALID;
    rr_status_t st0 = check_shape(R, count, 6, opt);
    if (st0 != RR_OK) return st0;
    if (!send || !recv) return RR_ERR_INVALID;
    if (count == 0) return RR_OK;
    const uint64_t es = elem_bytes(dt);
    const uint64_t bytes = (uint64_t)R * count * es;
    std::vector<std::pair<uintptr_t, uint64_t>> iv;
    for (int r = 0; r < R; ++r) {
        if (!send[r] || !recv[r]) return RR_ERR_INVALID;
        if ((uintptr_t)send[r] % 16 || (uintptr_t)recv[r] % 16) return RR_ERR_INVALID;
        iv.push_back({(uintptr_t)send[r], bytes});
        iv.push_back({(uintptr_t)recv[r], bytes});
    }
    std::sort(iv.begin(), iv.end());
    for (size_t i = 0; i + 1 < iv.size(); ++i)
        if (iv[i].first + iv[i].second > iv[i + 1].first) return RR_ERR_INVALID;
    DeviceState* d = nullptr;
    rr_status_t st = ensure_device(&d);
    if (st != RR_OK) return st;
    if (!(opt && (opt->flags & RR_FLAG_NO_POINTER_CHECK))) {
        if ((st = check_extents((void* const*)send, R, bytes)) != RR_OK) return st;
        if ((st = check_extents(recv, R, bytes)) != RR_OK) return st;
    }
    Plan p;
    if ((st = make_a2a_plan(d, R, count, dt, opt, &p)) != RR_OK) return st;
    A2AArgs a;
    memset(&a, 0, sizeof a);
    for (int r = 0; r < R; ++r) {
        a.send[r] = send[r];
        a.recv[r] = recv[r];
    }
    a.count = count;
    a.part_len = p.sub_len;
    a.sig = d->sig;        // receiver q uses slot q (lane 0 of the ring layout)
    a.shadow = d->shadow;
    a.err = d->err;
    a.timeout_ticks = timeout_ticks(d, opt);
    a.R = R;
    a.parts = p.cols;
    a.aligned = (count * es) % 16 == 0;
    a.inject = opt ? opt->inject : 0;
    hipStream_t s = (hipStream_t)stream;
    if (es == 2)
        hipLaunchKernelGGL((alltoall_kernel<2, kA2ABlock>), dim3(p.grid), dim3(kA2ABlock), 0, s, a);
    else
        hipLaunchKernelGGL((alltoall_kernel<4, kA2ABlock>), dim3(p.grid), dim3(kA2ABlock), 0, s, a);
    return hip_ok(hipGetLastError()) ? RR_OK : RR_ERR_HIP;
}

static rr_status_t fill(uint64_t* p, uint64_t n, uint64_t value, uint64_t stride, hipStream_t s) {
    if (n == 0) return RR_OK;
    const unsigned grid = (unsigned)std::min<uint64_t>(1024, ceil_div(n, 256));
    hipLaunchKernelGGL(fill_u64_kernel, dim3(grid), dim3(256), 0, s, p, n, value, stride);
    return hip_ok(hipGetLastError()) ? RR_OK : RR_ERR_HIP;
}

}  // namespace rr

using namespace rr;

struct rr_counting_barrier {
    int nwaiters;
    int ncontexts;
    int device;
    int pp_row;          // words per per-peer row: nwaiters rounded up to 128 bytes
    uint64_t* mem;       // one allocation holding the arrays below
    uint64_t* sig;       // counting signals, stride kSignalStride
    uint64_t* shadow;
    uint64_t* pp_sig;    // per-peer slots, one row per (context, waiter)
    uint64_t* pp_shadow;
    uint64_t* early;     // early passes seen by audited runs
};

extern "C" {

rr_status_t allreduce_ring_ex(void* const* bufs, int R, size_t count, rr_dtype_t dt, rr_op_t op,
                              int nslices, const rr_options_t* opt, rr_stream_t stream) {
    return run_ring(bufs, R, count, dt, op, nslices, 0, opt, stream);
}

rr_status_t reduce_scatter_ring_ex(void* const* bufs, int R, size_t count, rr_dtype_t dt,
                                   rr_op_t op, int nslices, const rr_options_t* opt,
                                   rr_stream_t stream) {
    return run_ring(bufs, R, count, dt, op, nslices, 1, opt, stream);
}

rr_status_t all_gather_ring_ex(void* const* bufs, int R, size_t count, rr_dtype_t dt, int nslices,
                               const rr_options_t* opt, rr_stream_t stream) {
    // A bit copy: the fold is never called, any op selects the same copy path.
    return run_ring(bufs, R, count, dt, RR_SUM, nslices, 2, opt, stream);
}

rr_status_t allreduce_ring(void* const* bufs, int R, size_t count, rr_dtype_t dt, rr_op_t op,
                           int nslices, rr_stream_t stream) {
    return run_ring(bufs, R, count, dt, op, nslices, 0, nullptr, stream);
}

rr_status_t reduce_scatter_ring(void* const* bufs, int R, size_t count, rr_dtype_t dt, rr_op_t op,
                                int nslices, rr_stream_t stream) {
    return run_ring(bufs, R, count, dt, op, nslices, 1, nullptr, stream);
}

rr_status_t all_gather_ring(void* const* bufs, int R, size_t count, rr_dtype_t dt, int nslices,
                            rr_stream_t stream) {
    return run_ring(bufs, R, count, dt, RR_SUM, nslices, 2, nullptr, stream);
}

rr_status_t allreduce_ring_staged(const void* const* sendbufs, void* const* recvbufs, int R,
                                  size_t count, rr_dtype_t dt, rr_op_t op, int nslices,
                                  const rr_options_t* opt, rr_stream_t stream) {
    return run_staged(sendbufs, recvbufs, R, count, dt, op, nslices, MODE_ALLREDUCE, opt, stream);
}

rr_status_t reduce_scatter(const void* const* sendbufs, void* const* recvbufs, int R,
                           size_t recvcount, rr_dtype_t dt, rr_op_t op, int nslices,
                           const rr_options_t* opt, rr_stream_t stream) {
    return run_staged(sendbufs, recvbufs, R, recvcount, dt, op, nslices, MODE_RS, opt, stream);
}

rr_status_t all_gather(const void* const* sendbufs, void* const* recvbufs, int R, size_t sendcount,
                       rr_dtype_t dt, int nslices, const rr_options_t* opt, rr_stream_t stream) {
    return run_staged(sendbufs, recvbufs, R, sendcount, dt, RR_SUM, nslices, MODE_AG, opt, stream);
}

rr_status_t alltoall(const void* const* sendbufs, void* const* recvbufs, int R, size_t count,
                     rr_dtype_t dt, const rr_options_t* opt, rr_stream_t stream) {
    return run_alltoall(sendbufs, recvbufs, R, count, dt, opt, stream);
}

rr_status_t rr_plan_query(int R, size_t count, rr_dtype_t dt, int nslices, int phase,
                          const rr_options_t* opt, rr_plan_t* out) {
    if (!out || phase < 0 || phase > 6) return RR_ERR_INVALID;
    if (R < 1 || R > RR_MAX_RANKS || nslices < 1 || nslices > RR_MAX_SLICES) return RR_ERR_INVALID;
    if (!valid_dtype(dt)) return RR_ERR_INVALID;
    rr_status_t st = check_shape(R, count, phase, opt);
    if (st != RR_OK) return st;
    DeviceState* d = nullptr;
    st = ensure_device(&d);
    if (st != RR_OK) return st;
    Plan p;
    if (phase <= 2)
        st = make_plan(d, R, count, dt, RR_SUM, nslices, phase, opt, &p);
    else if (phase <= 5)
        st = make_staged_plan(d, R, count, dt, RR_SUM, nslices, phase - 3, opt, &p);
    else
        st = make_a2a_plan(d, R, count, dt, opt, &p);
    if (st != RR_OK) return st;
    out->sync = p.sync;
    out->team = p.team;
    out->rounds = p.rounds;
    out->depth = p.depth;
    out->fused = p.fuse;
    out->stream_loads = p.stream_in;
    out->block = p.block;
    out->grid = p.grid;
    out->launches = (R == 1 || count == 0) ? 0 : p.launches;
    out->xcd_map = p.xcd_map;
    out->cooperative = p.coop;
    out->resident_max = p.resident_max;
    out->chunk_len = p.chunk_len;
    out->slice_len = p.slice_len;
    out->sub_len = p.sub_len;
    out->hbm_bytes = p.hbm_bytes;
    return RR_OK;
}

rr_status_t counting_barrier_create(int nwaiters, int ncontexts, rr_counting_barrier_t** out) {
    if (!out || nwaiters < 1 || nwaiters > RR_MAX_RANKS || ncontexts < 1 ||
        ncontexts > RR_MAX_SLICES)
        return RR_ERR_INVALID;
    *out = nullptr;
    int dev = 0;
    if (!hip_ok(hipGetDevice(&dev))) return RR_ERR_HIP;
    const size_t slots = (size_t)nwaiters * ncontexts;
    const int pp_row = (int)round_up((uint64_t)nwaiters, 16);
    const size_t words = slots * kSignalStride + slots + 2 * slots * pp_row + slots;
    void* p = nullptr;
    if (!hip_ok(hipMalloc(&p, words * sizeof(uint64_t)))) return RR_ERR_NOMEM;
    if (!hip_ok(hipMemset(p, 0, words * sizeof(uint64_t)))) {
        (void)hipFree(p);
        return RR_ERR_HIP;
    }
    rr_counting_barrier* b = (rr_counting_barrier*)calloc(1, sizeof(rr_counting_barrier));
    if (!b) {
        (void)hipFree(p);
        return RR_ERR_NOMEM;
    }
    b->nwaiters = nwaiters;
    b->ncontexts = ncontexts;
    b->device = dev;
    b->pp_row = pp_row;
    b->mem = (uint64_t*)p;
    b->sig = b->mem;
    b->shadow = b->sig + slots * kSignalStride;
    b->pp_sig = b->shadow + slots;
    b->pp_shadow = b->pp_sig + slots * pp_row;
    b->early = b->pp_shadow + slots * pp_row;
    *out = b;
    return RR_OK;
}

rr_status_t counting_barrier_destroy(rr_counting_barrier_t* b) {
    if (!b) return RR_OK;
    rr_status_t st = RR_OK;
    if (!hip_ok(hipDeviceSynchronize())) st = RR_ERR_HIP;
    if (!hip_ok(hipFree(b->mem))) st = RR_ERR_HIP;
    free(b);
    return st;
}

rr_status_t counting_barrier_preset(rr_counting_barrier_t* b, uint64_t value, rr_stream_t stream) {
    if (!b) return RR_ERR_INVALID;
    const uint64_t slots = (uint64_t)b->nwaiters * b->ncontexts;
    hipStream_t s = (hipStream_t)stream;
    rr_status_t st = fill(b->sig, slots, value, kSignalStride, s);
    if (st == RR_OK) st = fill(b->shadow, slots, value, 1, s);
    if (st == RR_OK) st = fill(b->pp_sig, 2 * slots * b->pp_row, value, 1, s);  // with shadows
    if (st == RR_OK) st = fill(b->early, slots, 0, 1, s);
    return st;
}

rr_status_t counting_barrier_reset(rr_counting_barrier_t* b, rr_stream_t stream) {
    return counting_barrier_preset(b, 0, stream);
}

rr_status_t counting_barrier_read(rr_counting_barrier_t* b, int ctx, int waiter, uint64_t* value,
                                  uint64_t* shadow) {
    if (!b || ctx < 0 || ctx >= b->ncontexts || waiter < 0 || waiter >= b->nwaiters)
        return RR_ERR_INVALID;
    if (!hip_ok(hipDeviceSynchronize())) return RR_ERR_HIP;
    const size_t slot = (size_t)ctx * b->nwaiters + waiter;
    uint64_t v = 0, sh = 0;
    if (!hip_ok(hipMemcpy(&v, b->sig + slot * kSignalStride, sizeof v, hipMemcpyDeviceToHost)))
        return RR_ERR_HIP;
    if (!hip_ok(hipMemcpy(&sh, b->shadow + slot, sizeof sh, hipMemcpyDeviceToHost)))
        return RR_ERR_HIP;
    if (value) *value = v;
    if (shadow) *shadow = sh;
    return RR_OK;
}

rr_status_t counting_barrier_read_peer(rr_counting_barrier_t* b, int ctx, int waiter, int peer,
                                       uint64_t* value, uint64_t* shadow) {
    if (!b || ctx < 0 || ctx >= b->ncontexts || waiter < 0 || waiter >= b->nwaiters ||
        peer < 0 || peer >= b->nwaiters || peer == waiter)
        return RR_ERR_INVALID;
    if (!hip_ok(hipDeviceSynchronize())) return RR_ERR_HIP;
    const size_t at = ((size_t)ctx * b->nwaiters + waiter) * b->pp_row + peer;
    uint64_t v = 0, sh = 0;
    if (!hip_ok(hipMemcpy(&v, b->pp_sig + at, sizeof v, hipMemcpyDeviceToHost))) return RR_ERR_HIP;
    if (!hip_ok(hipMemcpy(&sh, b->pp_shadow + at, sizeof sh, hipMemcpyDeviceToHost)))
        return RR_ERR_HIP;
    if (value) *value = v;
    if (shadow) *shadow = sh;
    return RR_OK;
}

rr_status_t counting_barrier_early_passes(rr_counting_barrier_t* b, int ctx, int waiter,
                                          uint64_t* count) {
    if (!b || !count || ctx < 0 || ctx >= b->ncontexts || waiter < 0 || waiter >= b->nwaiters)
        return RR_ERR_INVALID;
    if (!hip_ok(hipDeviceSynchronize())) return RR_ERR_HIP;
    const size_t at = (size_t)ctx * b->nwaiters + waiter;
    return hip_ok(hipMemcpy(count, b->early + at, sizeof *count, hipMemcpyDeviceToHost))
               ? RR_OK
               : RR_ERR_HIP;
}

static rr_status_t run_barrier(rr_counting_barrier_t* b, int R, int nsteps, int ncontexts,
                               uint64_t expected_per_step, const rr_options_t* opt,
                               uint64_t* stamps, rr_stream_t stream) {
    if (!b || R < 1 || R > b->nwaiters || ncontexts < 1 || ncontexts > b->ncontexts || nsteps < 0)
        return RR_ERR_INVALID;
    if (opt && (opt->sync < RR_SYNC_AUTO || opt->sync > RR_SYNC_PER_PEER)) return RR_ERR_INVALID;
    DeviceState* d = nullptr;
    rr_status_t st = ensure_device(&d);
    if (st != RR_OK) return st;
    const int grid = R * (int)round_up((uint64_t)ncontexts, 8);
    if (grid > resident_limit(d, (const void*)barrier_kernel, 64)) return RR_ERR_UNSUPPORTED;
    BarrierArgs a;
    memset(&a, 0, sizeof a);
    a.sig = b->sig;
    a.shadow = b->shadow;
    a.pp_sig = b->pp_sig;
    a.pp_shadow = b->pp_shadow;
    a.early = b->early;
    a.pp_row = b->pp_row;
    a.xcc_table = d->xcc_table;
    a.err = d->err;
    a.nctx = ncontexts;
    a.launch = {d->launch_gen, d->launch_exits};
    a.timeout_ticks = timeout_ticks(d, opt);
    a.expected = expected_per_step;
    a.R = R;
    a.stride = b->nwaiters;
    a.nsteps = nsteps;
    a.mode = !opt ? SYNC_BARRIER
                  : opt->sync == RR_SYNC_P2P ? SYNC_P2P
                  : opt->sync == RR_SYNC_PER_PEER ? SYNC_PER_PEER : SYNC_BARRIER;
    a.inject = opt ? opt->inject : 0;
    a.audit = opt && (opt->flags & RR_FLAG_AUDIT) ? 1 : 0;
    a.stamps = stamps;
    void* args[] = {&a};
    hipStream_t s = (hipStream_t)stream;
    const bool coop = opt && (opt->flags & RR_FLAG_COOPERATIVE);
    if (coop) {
        if (!hip_ok(hipLaunchCooperativeKernel((const void*)barrier_kernel, dim3(grid), dim3(64),
                                               args, 0, s))) {
            (void)hipGetLastError();
            return RR_ERR_HIP;
        }
    } else {
        hipLaunchKernelGGL(barrier_kernel, dim3(grid), dim3(64), 0, s, a);
    }
    return hip_ok(hipGetLastError()) ? RR_OK : RR_ERR_HIP;
}

rr_status_t counting_barrier_run(rr_counting_barrier_t* b, int R, int nsteps, int ncontexts,
                                 uint64_t expected_per_step, const rr_options_t* opt,
                                 rr_stream_t stream) {
    return run_barrier(b, R, nsteps, ncontexts, expected_per_step, opt, nullptr, stream);
}

rr_status_t counting_barrier_run_timed(rr_counting_barrier_t* b, int R, int nsteps,
                                       int ncontexts, uint64_t expected_per_step,
                                       const rr_options_t* opt, uint64_t* stamps,
                                       uint32_t* clock_khz, rr_stream_t stream) {
    if (!b || !stamps || !clock_khz || R < 1 || R > b->nwaiters || ncontexts < 1 ||
        ncontexts > b->ncontexts || nsteps < 0 || (uintptr_t)stamps % 8 != 0)
        return RR_ERR_INVALID;
    if (!(opt && (opt->flags & RR_FLAG_NO_POINTER_CHECK))) {
        void* const buf[1] = {stamps};
        const size_t bytes = (size_t)ncontexts * R * ((size_t)nsteps + 1) * sizeof(uint64_t);
        rr_status_t st = check_extents(buf, 1, bytes);
        if (st != RR_OK) return st;
    }
    DeviceState* d = nullptr;
    rr_status_t st = ensure_device(&d);
    if (st != RR_OK) return st;
    *clock_khz = (uint32_t)d->wall_khz;
    return run_barrier(b, R, nsteps, ncontexts, expected_per_step, opt, stamps, stream);
}

rr_status_t rr_last_kernel_error(rr_stream_t stream, rr_error_record_t* rec) {
    DeviceState* d = nullptr;
    rr_status_t st = ensure_device(&d);
    if (st != RR_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (!hip_ok(hipStreamSynchronize(s))) return RR_ERR_HIP;
    ErrorRecord e;
    if (!hip_ok(hipMemcpy(&e, d->err, sizeof e, hipMemcpyDeviceToHost))) return RR_ERR_HIP;
    if (rec) memset(rec, 0, sizeof *rec);
    if (e.flag == 0) return RR_OK;
    if (rec) {
        rec->status = e.status;
        rec->ctx = e.ctx;
        rec->waiter = e.waiter;
        rec->hop = e.hop;
        rec->peer = e.peer;
        rec->expected = e.expected;
        rec->observed = e.observed;
    }
    // clear the record and restore sig == shadow everywhere
    if ((st = fill(d->sig, kSlots, 0, kSignalStride, s)) != RR_OK) return st;
    if ((st = fill(d->shadow, kSlots, 0, 1, s)) != RR_OK) return st;
    if ((st = fill(d->credit, kSlots, 0, kSignalStride, s)) != RR_OK) return st;
    if ((st = fill(d->credit_shadow, kSlots, 0, 1, s)) != RR_OK) return st;
    if ((st = fill((uint64_t*)d->err, sizeof(ErrorRecord) / 8, 0, 1, s)) != RR_OK) return st;
    if (!hip_ok(hipStreamSynchronize(s))) return RR_ERR_HIP;
    return e.status == RR_ERR_TIMEOUT ? RR_ERR_TIMEOUT : RR_ERR_HIP;
}

rr_status_t rr_init(void) {
    DeviceState* d = nullptr;
    return ensure_device(&d);
}

rr_status_t rr_workspace_preset(uint64_t value, rr_stream_t stream) {
    DeviceState* d = nullptr;
    rr_status_t st = ensure_device(&d);
    if (st != RR_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if ((st = fill(d->sig, kSlots, value, kSignalStride, s)) != RR_OK) return st;
    if ((st = fill(d->shadow, kSlots, value, 1, s)) != RR_OK) return st;
    if ((st = fill(d->credit, kSlots, value, kSignalStride, s)) != RR_OK) return st;
    return fill(d->credit_shadow, kSlots, value, 1, s);
}

rr_status_t rr_hbm_copy(void* dst, const void* src, size_t bytes, rr_stream_t stream) {
    if (!dst || !src || (uintptr_t)dst % 16 || (uintptr_t)src % 16) return RR_ERR_INVALID;
    if (bytes == 0) return RR_OK;
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
    if (a < b + bytes && b < a + bytes) return RR_ERR_INVALID;
    DeviceState* d = nullptr;
    rr_status_t st = ensure_device(&d);
    if (st != RR_OK) return st;
    void* const ptrs[2] = {dst, (void*)src};
    if ((st = check_extents(ptrs, 2, bytes)) != RR_OK) return st;
    const uint64_t nvec = bytes / 16;
    const uint32_t ntail = (uint32_t)(bytes % 16);
    const unsigned grid = (unsigned)std::max<uint64_t>(
        1, std::min<uint64_t>((uint64_t)d->cus * kCopyPerCU, ceil_div(nvec, 8 * kCopyBlock)));
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(kCopyBlock), 0, (hipStream_t)stream,
                       (const u32x4*)src, (u32x4*)dst, nvec, (const uint8_t*)src + nvec * 16,
                       (uint8_t*)dst + nvec * 16, ntail);
    return hip_ok(hipGetLastError()) ? RR_OK : RR_ERR_HIP;
}

const char* rr_status_string(rr_status_t s) {
    switch (s) {
        case RR_OK: return "RR_OK";
        case RR_ERR_INVALID: return "RR_ERR_INVALID: invalid argument";
        case RR_ERR_UNSUPPORTED: return "RR_ERR_UNSUPPORTED: not supported by the requested mode";
        case RR_ERR_HIP: return "RR_ERR_HIP: HIP runtime error";
        case RR_ERR_TIMEOUT: return "RR_ERR_TIMEOUT: a device wait timed out";
        case RR_ERR_NOMEM: return "RR_ERR_NOMEM: out of memory";
    }
    return "unknown rr_status_t";
}

int rr_abi_version(void) { return RR_ABI_VERSION; }

void rr_finalize(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    for (int i = 0; i < kMaxDevices; ++i) {
        DeviceState& d = g_dev[i];
        if (!d.ready) continue;
        int prev = 0;
        (void)hipGetDevice(&prev);
        (void)hipSetDevice(i);
        (void)hipDeviceSynchronize();
        (void)hipFree(d.mem);
        if (d.fifo) (void)hipFree(d.fifo);
        (void)hipSetDevice(prev);
        d = DeviceState();
    }
}

}  // extern "C"
