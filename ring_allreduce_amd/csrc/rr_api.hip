// rr_api.hip -- the host side of the library: per-device workspace, plans,
// argument checks, launches, and the C ABI declared in include/rr.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "rr.h"
#include "rr_kernels.hpp"

namespace rr {

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
// long-ring rule.  One exception plans its columns for 1024 threads: a barrier
// per hop on a long ring with a wide hop (below).
constexpr int kAutoBlock = 512;
constexpr int kSmallBlock = 128;
constexpr int kMidBlock = 256;
constexpr uint64_t kTinyPieceBytes = 2ull << 10;
constexpr uint64_t kMidPieceLo = 16ull << 10;   // exclusive
constexpr uint64_t kMidPieceHi = 32ull << 10;
constexpr int kLongRingRanks = 16;
constexpr uint64_t kLongRingPieceBytes = 64ull << 10;
// A barrier per hop on a long ring whose hop moves at least 1.5 GiB over all
// ranks (512 MiB per rank and more) runs one 1024-thread workgroup per CU
// instead of two of 512, still two lanes per workgroup and the same bytes per
// round: fewer, larger pieces per barrier.  Measured on MI355X with interleaved
// repeats: +6.0% and +3.2% at 16 ranks x 512 MiB and 1 GiB, +1.0% and +3.1% at
// 32 ranks; within +-1% at 256 MiB per rank and with predecessor hand-offs, and
// worse at 8 ranks, so only this case takes it.  It needs whole columns of 8
// (8 R dividing the CU count: 16 and 32 ranks on 256 CUs).
constexpr uint64_t kWideBarrierHopBytes = 1536ull << 20;
constexpr int kWideBarrierBlock = 1024;

// ------------------------------------------------------------- host side --

struct DeviceState {
    bool info = false;    // attributes below read
    bool ready = false;   // workspace allocated
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
    std::vector<void*> retired;         // receive buffers outgrown, kept until rr_finalize
    uint64_t* launch_gen = nullptr;     // per-launch tag of the XCD table (starts at 1)
    uint64_t* launch_exits = nullptr;   // workgroups of the running launch that have left
    uint64_t* lane_sig = nullptr;       // barrier: one signal per lane (unless RR_FLAG_WAITER_SIGNAL)
    uint64_t* lane_shadow = nullptr;
    // resident workgroups per CU of each kernel handle, as the occupancy query
    // answered it (asked once per kernel and device, not once per call)
    std::vector<std::pair<const void*, int>> occupancy;
};

std::mutex g_mu;
DeviceState g_dev[kMaxDevices];

struct Plan {
    int nap;
    int stream_in;
    int alternate;
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

// The current device's attributes (compute units, wall-clock rate).  Allocates
// nothing.  Call with g_mu held.
static rr_status_t device_info_locked(int dev, DeviceState& d) {
    if (d.info) return RR_OK;
    if (!hip_ok(hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev)))
        return RR_ERR_HIP;
    if (!hip_ok(hipDeviceGetAttribute(&d.wall_khz, hipDeviceAttributeWallClockRate, dev)) ||
        d.wall_khz <= 0)
        d.wall_khz = 100000;  // the gfx9 constant-rate clock runs at 100 MHz
    d.info = true;
    return RR_OK;
}

static rr_status_t current_device(int* dev) {
    if (!hip_ok(hipGetDevice(dev))) return RR_ERR_HIP;
    if (*dev < 0 || *dev >= kMaxDevices) return RR_ERR_UNSUPPORTED;
    return RR_OK;
}

static rr_status_t ensure_device(DeviceState** out) {
    int dev = 0;
    rr_status_t st = current_device(&dev);
    if (st != RR_OK) return st;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState& d = g_dev[dev];
    if (!d.ready) {
        if ((st = device_info_locked(dev, d)) != RR_OK) return st;
        // signals (one per cache line), shadows, the XCC table, the error record,
        // the staged loop's credit signals and their shadows, then the launch tag
        // and the exit count (a cache line each)
        const size_t words = 3 * ((size_t)kSlots * kSignalStride + (size_t)kSlots) +
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
        d.lane_sig = d.launch_exits + kSignalStride;
        d.lane_shadow = d.lane_sig + (size_t)kSlots * kSignalStride;
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
    // flags that exclude each other
    if ((opt->flags & RR_FLAG_SHARED_SIGNAL) && (opt->flags & RR_FLAG_WAITER_SIGNAL))
        return RR_ERR_INVALID;
    if ((opt->flags & RR_FLAG_ASCENDING) && (opt->flags & RR_FLAG_ALTERNATE))
        return RR_ERR_INVALID;
    const uint32_t polls =
        opt->flags & (RR_FLAG_POLL_FAST | RR_FLAG_POLL_MEDIUM | RR_FLAG_POLL_SLOW);
    if (polls & (polls - 1)) return RR_ERR_INVALID;
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
// kernel can touch memory outside what the caller handed over.  Buffers inside
// an allocation already checked in this call (rank buffers carved from one
// allocation) need no further runtime query.
static rr_status_t check_extents(void* const* bufs, int R, size_t bytes) {
    int dev = 0;
    if (!hip_ok(hipGetDevice(&dev))) return RR_ERR_HIP;
    uintptr_t seen_lo[8], seen_hi[8];
    int nseen = 0;
    for (int r = 0; r < R; ++r) {
        const uintptr_t b = (uintptr_t)bufs[r];
        bool inside = false;
        for (int k = 0; k < nseen && !inside; ++k)
            inside = b >= seen_lo[k] && b <= seen_hi[k] && bytes <= seen_hi[k] - b;
        if (inside) continue;
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
        if (nseen < 8) {
            seen_lo[nseen] = (uintptr_t)base;
            seen_hi[nseen] = (uintptr_t)base + size;
            ++nseen;
        }
    }
    return RR_OK;
}

// Workgroups of `kernel` (one instantiation per workgroup size) the device can
// hold at once.  The answer is fixed per kernel and device, so it is kept.
static int resident_limit(const DeviceState* d, const void* kernel, int block) {
    {
        std::lock_guard<std::mutex> lock(g_mu);
        for (const auto& e : d->occupancy)
            if (e.first == kernel) return e.second * d->cus;
    }
    int per_cu = 0;
    if (!hip_ok(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0))) {
        (void)hipGetLastError();
        return 0;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    const_cast<DeviceState*>(d)->occupancy.push_back({kernel, per_cu});
    return per_cu * d->cus;
}

// phase: 0 AllReduce, 1 ReduceScatter, 2 AllGather.
static rr_status_t make_plan(const DeviceState* d, int R, size_t count, int dt, int op,
                             int nslices, int phase, const rr_options_t* opt, Plan* p) {
    const uint64_t V = 16 / elem_bytes(dt);
    const bool fixed_block = opt && opt->block;
    int block = fixed_block ? opt->block : kAutoBlock;
    const int requested = opt ? opt->sync : RR_SYNC_AUTO;
    const bool barrier = requested == RR_SYNC_BARRIER;
    const uint64_t hop_bytes = 3ull * (uint64_t)count * elem_bytes(dt);
    const bool wide_barrier = !fixed_block && barrier && R >= kLongRingRanks &&
                              hop_bytes >= kWideBarrierHopBytes && d->cus % (8 * R) == 0;
    if (wide_barrier) block = kWideBarrierBlock;
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
    // workgroups (one of 1024 for a wide barrier hop).  Each interleaves `depth` lanes and runs `rounds` groups of
    // them one after another; rounds bound one hop of the lanes in flight
    // (3 N / rounds bytes over all ranks), so that a partial is still cached
    // when the next hop reads it.
    const int target_cols = std::max(1, d->cus * 16 * 64 / block / R);
    const bool fixed_depth = opt && opt->depth > 0;
    const bool fixed_rounds = opt && opt->rounds > 0;
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
    if (!fixed_block && !wide_barrier) {
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
    // even hops top down once the buffers outgrow half the Infinity Cache: a hop
    // then reads first what its predecessor wrote last (A/B over R = 2-64 and
    // 1 MiB-1 GiB per rank: +0.5-3% above, up to 3% slower at 64-128 MiB in all).
    // It is a kernel of its own, so that the smaller calls keep the leaner code.
    p->alternate = (flags & RR_FLAG_ALTERNATE) ||
                   (!(flags & RR_FLAG_ASCENDING) && (uint64_t)R * nbytes > kInfinityCacheBytes / 2);
    const void* kernel = (const void*)pick_ring_kernel(dt, op, block, p->alternate != 0);
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
    p->nap = sync == RR_SYNC_BARRIER && 3ull * count * elem_bytes(dt) >= kLongNapBytes ? 2 : 0;
    if (flags & RR_FLAG_POLL_FAST) p->nap = 0;
    if (flags & RR_FLAG_POLL_MEDIUM) p->nap = 1;
    if (flags & RR_FLAG_POLL_SLOW) p->nap = 2;
    p->stream_in = (flags & RR_FLAG_STREAM_LOADS) ||
                   (!(flags & RR_FLAG_CACHED_LOADS) && (uint64_t)R * nbytes > kInfinityCacheBytes);
    return RR_OK;
}

// stamps: optional per-hop clock stamps (allreduce_ring_timed), stamp_words long.
static rr_status_t run_ring(void* const* bufs, int R, size_t count, int dt, int op, int nslices,
                            int phase, const rr_options_t* opt, rr_stream_t stream,
                            uint64_t* stamps = nullptr, size_t stamp_words = 0) {
    rr_status_t st = check_args(bufs, R, count, dt, op, nslices, opt);
    if (st != RR_OK || R == 1 || count == 0) return st;
    DeviceState* d = nullptr;
    if ((st = ensure_device(&d)) != RR_OK) return st;
    const bool checked = !(opt && (opt->flags & RR_FLAG_NO_POINTER_CHECK));
    if (checked)
        if ((st = check_extents(bufs, R, count * elem_bytes(dt))) != RR_OK) return st;
    Plan p;
    if ((st = make_plan(d, R, count, dt, op, nslices, phase, opt, &p)) != RR_OK) return st;
    if (stamps) {
        // 3 words per (lane, rank, hop of the whole AllReduce)
        const uint64_t need = (uint64_t)nslices * p.team * R * (2ull * (R - 1)) * 3;
        if (stamp_words < need) return RR_ERR_INVALID;
        if (checked) {
            void* const sb[1] = {stamps};
            if ((st = check_extents(sb, 1, (size_t)need * sizeof(uint64_t))) != RR_OK) return st;
        }
    }

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
    a.nap = p.nap;
    a.stream_in = p.stream_in;
    // a barrier per hop: one signal per lane shared by all R ranks, unless the
    // caller asks for one signal per waiter
    a.shared_sig = p.sync == RR_SYNC_BARRIER && !(opt && (opt->flags & RR_FLAG_WAITER_SIGNAL)) ? 1 : 0;
    a.lane_sig = d->lane_sig;
    a.lane_shadow = d->lane_shadow;
    a.stamps = stamps;
    a.xcd_map = p.xcd_map;
    a.inject = opt ? opt->inject : 0;
    RingKernel k = pick_ring_kernel(dt, op, p.block, p.alternate != 0);
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
// slots: (lane, rank) signal slots available, which also bounds the grid (the
// XCD table has one entry per slot).
static rr_status_t make_staged_plan(const DeviceState* d, int R, uint64_t n, int dt, int op,
                                    int nslices, int mode, const rr_options_t* opt, Plan* p,
                                    int slots = kSlots) {
    const uint64_t es = elem_bytes(dt);
    const uint64_t V = 16 / es;
    const int requested = opt ? opt->sync : RR_SYNC_AUTO;
    const uint32_t flags = opt ? opt->flags : 0;
    if (opt && opt->block != 0 && opt->block != kStagedBlock) return RR_ERR_UNSUPPORTED;
    if (requested == RR_SYNC_BARRIER) return RR_ERR_UNSUPPORTED;  // credits pace the loop
    p->block = kStagedBlock;
    p->fuse = 0;
    p->stream_in = 0;
    p->alternate = 0;
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
    const int max_team = std::max(1, slots / (R * nslices));
    if (team > max_team) {
        if (opt && opt->team > 0) return RR_ERR_UNSUPPORTED;
        team = max_team;
    }
    const int lanes = nslices * team;
    if ((int64_t)lanes * R > slots) return RR_ERR_UNSUPPORTED;
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
    if (sync == RR_SYNC_P2P && (p->grid > p->resident_max || p->grid > slots))
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

// Grows the staged loop's receive buffers.  An outgrown buffer is not freed
// until rr_finalize: kernels still queued, and launches captured earlier into a
// HIP graph, hold its address.
static rr_status_t ensure_fifo(DeviceState* d, size_t bytes) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (d->fifo_bytes >= bytes) return RR_OK;
    void* p = nullptr;
    if (!hip_ok(hipMalloc(&p, bytes))) return RR_ERR_NOMEM;
    if (d->fifo) d->retired.push_back(d->fifo);
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
    hipLaunchKernelGGL(copy_kernel_handle(), dim3(grid), dim3(kCopyBlock), 0, s, (const u32x4*)src, (u32x4*)dst,
                       nvec, (const uint8_t*)src + nvec * 16, (uint8_t*)dst + nvec * 16, ntail);
    return hip_ok(hipGetLastError()) ? RR_OK : RR_ERR_HIP;
}

// ------------------------------------------ the staged loop without allocation
//
// allreduce_ring_staged_noalloc keeps everything the staged kernel needs beyond
// the caller's buffers -- receive slots, ready and credit signals with their
// shadows, the XCD table, the failure record, the launch tag -- in `scratch`, a
// device array of fixed size in this library's code object.  Zeroed memory is a
// valid starting state (every signal equals its shadow, no failure recorded,
// table entries unpublished), so nothing is written at set-up.  In host code
// `scratch` names a host-side stand-in; its device address, one per device, comes
// from hipGetSymbolAddress and is the only address ever handed to a kernel.
constexpr int kScratchSlots = 4096;                       // (lane, rank) pairs
constexpr uint64_t kScratchFifoBytes = 64ull << 20;       // receive slots
constexpr size_t kScratchFifoWords = kScratchFifoBytes / 8;
constexpr size_t kScratchSignalWords = (size_t)kScratchSlots * kSignalStride;
constexpr size_t kScratchWords = kScratchFifoWords          // receive slots (first: aligned)
                                 + 2 * kScratchSignalWords  // ready and credit signals
                                 + 2 * (size_t)kScratchSlots  // their shadows
                                 + (size_t)kScratchSlots    // XCD table
                                 + 16                       // failure record
                                 + 2 * (size_t)kSignalStride;  // launch tag, exit count

static __device__ __align__(256) uint64_t scratch[kScratchWords];

struct Scratch {
    char* fifo;
    uint64_t* ready;
    uint64_t* credit;
    uint64_t* ready_shadow;
    uint64_t* credit_shadow;
    uint64_t* xcc_table;
    ErrorRecord* err;
    uint64_t* launch_gen;
    uint64_t* launch_exits;
};

uint64_t* g_scratch[kMaxDevices];  // device address of `scratch`, per device

static Scratch carve(uint64_t* base) {
    Scratch c;
    c.fifo = (char*)base;
    c.ready = base + kScratchFifoWords;
    c.credit = c.ready + kScratchSignalWords;
    c.ready_shadow = c.credit + kScratchSignalWords;
    c.credit_shadow = c.ready_shadow + kScratchSlots;
    c.xcc_table = c.credit_shadow + kScratchSlots;
    c.err = (ErrorRecord*)(c.xcc_table + kScratchSlots);
    c.launch_gen = c.xcc_table + kScratchSlots + 16;
    c.launch_exits = c.launch_gen + kSignalStride;
    return c;
}

// Looks up the device address of `scratch` on the current device once (with
// that device current) and keeps it.  Allocates nothing.  Call with g_mu held.
static rr_status_t scratch_locked(int dev, uint64_t** out) {
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (!hip_ok(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) || !p) {
            (void)hipGetLastError();
            return RR_ERR_HIP;
        }
        g_scratch[dev] = (uint64_t*)p;
    }
    *out = g_scratch[dev];
    return RR_OK;
}

static rr_status_t run_staged(const void* const* send, void* const* recv, int R, uint64_t n, int dt,
                              int op, int nslices, int mode, const rr_options_t* opt,
                              rr_stream_t stream, bool noalloc = false) {
    rr_status_t st = check_staged_args(send, recv, R, n, dt, op, nslices, mode, opt);
    if (st != RR_OK || n == 0) return st;
    DeviceState* d = nullptr;
    Scratch sc;
    memset(&sc, 0, sizeof sc);
    if (noalloc) {
        int dev = 0;
        if ((st = current_device(&dev)) != RR_OK) return st;
        std::lock_guard<std::mutex> lock(g_mu);
        if ((st = device_info_locked(dev, g_dev[dev])) != RR_OK) return st;
        uint64_t* base = nullptr;
        if ((st = scratch_locked(dev, &base)) != RR_OK) return st;
        d = &g_dev[dev];
        sc = carve(base);
    } else if ((st = ensure_device(&d)) != RR_OK) {
        return st;
    }
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
    if ((st = make_staged_plan(d, R, n, dt, op, nslices, mode, opt, &p,
                               noalloc ? kScratchSlots : kSlots)) != RR_OK)
        return st;
    const uint64_t slot_len = round_up(p.chunk_len, 16 / es);
    const uint64_t fifo_bytes = (uint64_t)R * kFifoSlots * slot_len * es;
    if (noalloc) {
        if (fifo_bytes > kScratchFifoBytes) return RR_ERR_UNSUPPORTED;
    } else if ((st = ensure_fifo(d, (size_t)fifo_bytes)) != RR_OK) {
        return st;
    }

    StagedArgs a;
    memset(&a, 0, sizeof a);
    for (int r = 0; r < R; ++r) {
        a.send[r] = send[r];
        a.recv[r] = recv[r];
    }
    a.slot_len = slot_len;
    a.n = n;
    a.chunk_len = p.chunk_len;
    a.slice_len = p.slice_len;
    a.sub_len = p.sub_len;
    if (noalloc) {
        a.fifo = sc.fifo;
        a.ready = sc.ready;
        a.ready_shadow = sc.ready_shadow;
        a.credit = sc.credit;
        a.credit_shadow = sc.credit_shadow;
        a.xcc_table = sc.xcc_table;
        a.err = sc.err;
        a.launch = {sc.launch_gen, sc.launch_exits};
    } else {
        a.fifo = d->fifo;
        a.ready = d->sig;
        a.ready_shadow = d->shadow;
        a.credit = d->credit;
        a.credit_shadow = d->credit_shadow;
        a.xcc_table = d->xcc_table;
        a.err = d->err;
        a.launch = {d->launch_gen, d->launch_exits};
    }
    a.timeout_ticks = timeout_ticks(d, opt);
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
    const void* kernel = (const void*)pick_alltoall_kernel((int)es);
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
    p->alternate = 0;
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
    AlltoallKernel k = pick_alltoall_kernel((int)es);
    hipLaunchKernelGGL(k, dim3(p.grid), dim3(kA2ABlock), 0, s, a);
    return hip_ok(hipGetLastError()) ? RR_OK : RR_ERR_HIP;
}

static rr_status_t fill(uint64_t* p, uint64_t n, uint64_t value, uint64_t stride, hipStream_t s) {
    if (n == 0) return RR_OK;
    const unsigned grid = (unsigned)std::min<uint64_t>(1024, ceil_div(n, 256));
    FillKernel k = fill_kernel_handle();
    hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, s, p, n, value, stride);
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
    uint64_t* ctx_sig;   // shared layout: one signal per context, stride kSignalStride
    uint64_t* ctx_shadow;
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

rr_status_t allreduce_ring_timed(void* const* bufs, int R, size_t count, rr_dtype_t dt, rr_op_t op,
                                 int nslices, const rr_options_t* opt, uint64_t* stamps,
                                 size_t stamp_words, uint32_t* clock_khz, rr_stream_t stream) {
    if (!stamps || !clock_khz || (uintptr_t)stamps % 8 != 0) return RR_ERR_INVALID;
    DeviceState* d = nullptr;
    rr_status_t st = ensure_device(&d);
    if (st != RR_OK) return st;
    *clock_khz = (uint32_t)d->wall_khz;
    return run_ring(bufs, R, count, dt, op, nslices, 0, opt, stream, stamps, stamp_words);
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

rr_status_t allreduce_ring_staged_noalloc(const void* const* sendbufs, void* const* recvbufs,
                                          int R, size_t count, rr_dtype_t dt, rr_op_t op,
                                          int nslices, const rr_options_t* opt,
                                          rr_stream_t stream) {
    return run_staged(sendbufs, recvbufs, R, count, dt, op, nslices, MODE_ALLREDUCE, opt, stream,
                      true);
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
    out->alternate = p.alternate;
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
    const size_t words = slots * kSignalStride + slots + 2 * slots * pp_row + slots +
                         (size_t)ncontexts * kSignalStride + (size_t)ncontexts;
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
    b->ctx_sig = b->early + slots;
    b->ctx_shadow = b->ctx_sig + (size_t)ncontexts * kSignalStride;
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
    if (st == RR_OK) st = fill(b->ctx_sig, (uint64_t)b->ncontexts, value, kSignalStride, s);
    if (st == RR_OK) st = fill(b->ctx_shadow, (uint64_t)b->ncontexts, value, 1, s);
    return st;
}

rr_status_t counting_barrier_reset(rr_counting_barrier_t* b, rr_stream_t stream) {
    return counting_barrier_preset(b, 0, stream);
}

rr_status_t counting_barrier_read(rr_counting_barrier_t* b, int ctx, int waiter, uint64_t* value,
                                  uint64_t* shadow) {
    if (!b || ctx < 0 || ctx >= b->ncontexts || waiter < -1 || waiter >= b->nwaiters)
        return RR_ERR_INVALID;
    if (!hip_ok(hipDeviceSynchronize())) return RR_ERR_HIP;
    const size_t slot = (size_t)ctx * b->nwaiters + waiter;
    // waiter -1: the context's shared signal and its shadow
    const uint64_t* vp = waiter < 0 ? b->ctx_sig + (size_t)ctx * kSignalStride
                                    : b->sig + slot * kSignalStride;
    const uint64_t* sp = waiter < 0 ? b->ctx_shadow + ctx : b->shadow + slot;
    uint64_t v = 0, sh = 0;
    if (!hip_ok(hipMemcpy(&v, vp, sizeof v, hipMemcpyDeviceToHost))) return RR_ERR_HIP;
    if (!hip_ok(hipMemcpy(&sh, sp, sizeof sh, hipMemcpyDeviceToHost))) return RR_ERR_HIP;
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
    BarrierKernel k = barrier_kernel_handle();
    if (grid > resident_limit(d, (const void*)k, 64)) return RR_ERR_UNSUPPORTED;
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
    a.shared = opt && (opt->flags & RR_FLAG_SHARED_SIGNAL) ? 1 : 0;
    a.ctx_sig = b->ctx_sig;
    a.ctx_shadow = b->ctx_shadow;
    a.stamps = stamps;
    void* args[] = {&a};
    hipStream_t s = (hipStream_t)stream;
    const bool coop = opt && (opt->flags & RR_FLAG_COOPERATIVE);
    if (coop) {
        if (!hip_ok(hipLaunchCooperativeKernel((const void*)k, dim3(grid), dim3(64),
                                               args, 0, s))) {
            (void)hipGetLastError();
            return RR_ERR_HIP;
        }
    } else {
        hipLaunchKernelGGL(k, dim3(grid), dim3(64), 0, s, a);
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

// Reads a failure record; if set, copies it out and clears it together with the
// signals and shadows of the workspace it belongs to.
static rr_status_t take_record(ErrorRecord* err, uint64_t* sig, uint64_t* shadow, uint64_t* credit,
                               uint64_t* credit_shadow, int slots, hipStream_t s, ErrorRecord* out,
                               bool* found) {
    ErrorRecord e;
    if (!hip_ok(hipMemcpy(&e, err, sizeof e, hipMemcpyDeviceToHost))) return RR_ERR_HIP;
    *found = e.flag != 0;
    if (!*found) return RR_OK;
    *out = e;
    rr_status_t st;
    if ((st = fill(sig, (uint64_t)slots, 0, kSignalStride, s)) != RR_OK) return st;
    if ((st = fill(shadow, (uint64_t)slots, 0, 1, s)) != RR_OK) return st;
    if ((st = fill(credit, (uint64_t)slots, 0, kSignalStride, s)) != RR_OK) return st;
    if ((st = fill(credit_shadow, (uint64_t)slots, 0, 1, s)) != RR_OK) return st;
    if ((st = fill((uint64_t*)err, sizeof(ErrorRecord) / 8, 0, 1, s)) != RR_OK) return st;
    return hip_ok(hipStreamSynchronize(s)) ? RR_OK : RR_ERR_HIP;
}

rr_status_t rr_last_kernel_error(rr_stream_t stream, rr_error_record_t* rec) {
    int dev = 0;
    rr_status_t st = current_device(&dev);
    if (st != RR_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (!hip_ok(hipStreamSynchronize(s))) return RR_ERR_HIP;
    DeviceState* d = nullptr;
    uint64_t* base = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        if (g_dev[dev].ready) d = &g_dev[dev];
        base = g_scratch[dev];
    }
    if (rec) memset(rec, 0, sizeof *rec);
    ErrorRecord e;
    memset(&e, 0, sizeof e);
    bool found = false;
    // the library-owned workspace, if one exists (nothing is allocated here)
    if (d && (st = take_record(d->err, d->sig, d->shadow, d->credit, d->credit_shadow, kSlots, s,
                               &e, &found)) != RR_OK)
        return st;
    if (d && found) {
        if ((st = fill(d->lane_sig, kSlots, 0, kSignalStride, s)) != RR_OK) return st;
        if ((st = fill(d->lane_shadow, kSlots, 0, 1, s)) != RR_OK) return st;
        if (!hip_ok(hipStreamSynchronize(s))) return RR_ERR_HIP;
    }
    // the static scratch of allreduce_ring_staged_noalloc, if it was used
    if (!found && base) {
        const Scratch c = carve(base);
        if ((st = take_record(c.err, c.ready, c.ready_shadow, c.credit, c.credit_shadow,
                              kScratchSlots, s, &e, &found)) != RR_OK)
            return st;
    }
    if (!found) return RR_OK;
    if (rec) {
        rec->status = e.status;
        rec->ctx = e.ctx;
        rec->waiter = e.waiter;
        rec->hop = e.hop;
        rec->peer = e.peer;
        rec->expected = e.expected;
        rec->observed = e.observed;
    }
    return e.status == RR_ERR_TIMEOUT ? RR_ERR_TIMEOUT : RR_ERR_HIP;
}

rr_status_t rr_init(void) {
    DeviceState* d = nullptr;
    rr_status_t st = ensure_device(&d);
    if (st != RR_OK) return st;
    int dev = 0;
    if ((st = current_device(&dev)) != RR_OK) return st;
    std::lock_guard<std::mutex> lock(g_mu);
    uint64_t* base = nullptr;
    return scratch_locked(dev, &base);
}

rr_status_t rr_workspace_preset(uint64_t value, rr_stream_t stream) {
    DeviceState* d = nullptr;
    rr_status_t st = ensure_device(&d);
    if (st != RR_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if ((st = fill(d->sig, kSlots, value, kSignalStride, s)) != RR_OK) return st;
    if ((st = fill(d->shadow, kSlots, value, 1, s)) != RR_OK) return st;
    if ((st = fill(d->credit, kSlots, value, kSignalStride, s)) != RR_OK) return st;
    if ((st = fill(d->lane_sig, kSlots, value, kSignalStride, s)) != RR_OK) return st;
    if ((st = fill(d->lane_shadow, kSlots, value, 1, s)) != RR_OK) return st;
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
    hipLaunchKernelGGL(copy_kernel_handle(), dim3(grid), dim3(kCopyBlock), 0, (hipStream_t)stream,
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
        for (void* q : d.retired) (void)hipFree(q);
        (void)hipSetDevice(prev);
        d = DeviceState();
    }
}

}  // extern "C"
