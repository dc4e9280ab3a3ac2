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
constexpr int kSlots = RR_MAX_SLICES * RR_MAX_RANKS;  // (context, rank) pairs
constexpr uint64_t kDefaultTimeoutNs = 2000000000ull;

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
    uint32_t generation; // per-launch tag, never 0
    int32_t pad0;
    int32_t R;
    int32_t team;
    int32_t g_first;     // hops run by this launch, 1-based, inclusive
    int32_t g_last;
    int32_t sync;        // SYNC_NONE (one hop per launch), SYNC_P2P, SYNC_BARRIER
    int32_t xcd_map;
    uint32_t inject;
    int32_t pad;
};

__device__ __forceinline__ uint64_t umin(uint64_t a, uint64_t b) { return a < b ? a : b; }

__device__ __forceinline__ int wrap(int a, int m) {
    const int r = a % m;
    return r < 0 ? r + m : r;
}

// Workgroup index of (rank k, lane) -- the inverse of the decoding in ring_kernel.
__device__ __forceinline__ int block_of(int k, int lane, int R, bool xcd_map) {
    return xcd_map ? ((lane >> 3) * R + k) * 8 + (lane & 7) : lane * R + k;
}

// The XCD (accelerator complex die) this wave runs on.
__device__ __forceinline__ uint32_t xcc_id() {
    return __builtin_amdgcn_s_getreg(20 /* HW_REG_XCC_ID */ | (0 << 6) | ((4 - 1) << 11));
}

// Called by wave 0.  True when all R workgroups of `lane` run on this
// workgroup's XCD, read from the table every workgroup fills at start; such a
// lane shares one L2, which then is the point where producer stores and
// consumer loads meet.  Every workgroup of the lane computes the same answer.
// Returns -1 if a lane-mate never published (timeout or a failure elsewhere).
__device__ int lane_on_one_xcd(const RingArgs& a, int lane, uint32_t mine) {
    const int k = threadIdx.x;
    int same = 1;
    int failed = 0;
    if (k < a.R) {
        const uint64_t* e = &a.xcc_table[block_of(k, lane, a.R, a.xcd_map != 0)];
        uint64_t v = sig_read(e);
        const uint64_t start = wall_clock64();
        uint32_t spins = 0;
        while ((uint32_t)(v >> 8) != a.generation) {
            __builtin_amdgcn_s_sleep(1);
            v = sig_read(e);
            if ((++spins & 31u) == 0u &&
                (sig_read(&a.err->flag) != 0 || wall_clock64() - start > a.timeout_ticks)) {
                failed = 1;
                break;
            }
        }
        same = !failed && (uint32_t)(v & 0xFFu) == mine;
    }
    if (__any(failed)) return -1;
    return __all(same) ? 1 : 0;
}

// One hop of one workgroup over elements [lo, hi) of both buffers.  ReduceScatter:
// dst = fold(src, dst).  AllGather: dst = src, bit for bit.  16-byte vectors,
// U vectors per thread in flight, then a scalar tail (only at the ragged end).
template <int DT, int OP, int BLOCK, int U>
__device__ __forceinline__ void hop_body(bool reduce, const void* srcbuf, void* dstbuf,
                                         uint64_t lo, uint64_t hi) {
    constexpr int ES = ElemBytes<DT>::value;
    constexpr int V = 16 / ES;
    const uint64_t n = hi - lo;
    const uint32_t nv = (uint32_t)(n / V);
    const u32x4* __restrict__ s = (const u32x4*)((const char*)srcbuf + lo * ES);
    u32x4* __restrict__ d = (u32x4*)((char*)dstbuf + lo * ES);
    uint32_t i = threadIdx.x;
    if (reduce) {
        for (; i + (U - 1) * BLOCK < nv; i += U * BLOCK) {
            u32x4 x[U], y[U];
#pragma unroll
            for (int u = 0; u < U; ++u) x[u] = s[i + u * BLOCK];
#pragma unroll
            for (int u = 0; u < U; ++u) y[u] = d[i + u * BLOCK];
#pragma unroll
            for (int u = 0; u < U; ++u) d[i + u * BLOCK] = fold4<DT, OP>(x[u], y[u]);
        }
        for (; i < nv; i += BLOCK) d[i] = fold4<DT, OP>(s[i], d[i]);
    } else {
        constexpr int UC = 2 * U;
        for (; i + (UC - 1) * BLOCK < nv; i += UC * BLOCK) {
            u32x4 x[UC];
#pragma unroll
            for (int u = 0; u < UC; ++u) x[u] = s[i + u * BLOCK];
#pragma unroll
            for (int u = 0; u < UC; ++u) d[i + u * BLOCK] = x[u];
        }
        for (; i < nv; i += BLOCK) d[i] = s[i];
    }
    const uint64_t t = (uint64_t)nv * V + threadIdx.x;  // fewer than V elements remain
    if (t < n) {
        const char* sp = (const char*)srcbuf + (lo + t) * ES;
        char* dp = (char*)dstbuf + (lo + t) * ES;
        if (reduce) {
            fold_one<DT, OP>(sp, dp);
        } else if (ES == 2) {
            *(uint16_t*)dp = *(const uint16_t*)sp;
        } else {
            *(uint32_t*)dp = *(const uint32_t*)sp;
        }
    }
}

template <int DT, int OP, int BLOCK>
__global__ void __launch_bounds__(BLOCK) ring_kernel(const RingArgs a) {
    constexpr int U = 4;
    const int R = a.R;
    int r, lane;
    if (a.xcd_map) {
        // Workgroups are dealt to the 8 XCDs round-robin by index; keep all R
        // ranks of a lane (slice j, member w) on one XCD so each hand-off stays
        // inside one L2.
        const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
        r = k % R;
        lane = (k / R) * 8 + x;
    } else {
        r = blockIdx.x % R;
        lane = blockIdx.x / R;
    }
    const int j = lane / a.team;
    const int w = lane - j * a.team;
    const int succ = r + 1 == R ? 0 : r + 1;
    const bool synced = a.g_last > a.g_first;
    const int my_slot = lane * R + r;

    __shared__ int s_stop;
    __shared__ int s_local;
    uint64_t shadow = 0;
    const uint32_t my_xcc = xcc_id() & 0xFu;
    if (threadIdx.x == 0) {
        s_stop = sig_read(&a.err->flag) != 0;  // a recorded failure is sticky
        if (synced) {
            shadow = a.shadow[my_slot];
            __hip_atomic_store(&a.xcc_table[blockIdx.x], ((uint64_t)a.generation << 8) | my_xcc,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    if (s_stop) return;
    // Producer side of the hand-off, fixed at the first hand-off of the launch:
    // local -- all R workgroups of the lane run on one XCD and so share its L2,
    //          the point where their loads and stores meet: each wave only waits
    //          until its stores have reached L2;
    // else  -- each wave makes its stores visible device-wide (agent-scope
    //          release: an L2 write-back), as a consumer may sit on another XCD.
    // The consumer side is the same in both cases: after the wait, one wave
    // performs an agent-scope acquire, which also invalidates the CU's L1.  That
    // matters even within one XCD: a workgroup re-reads a chunk of its incoming
    // buffer (the partial in ReduceScatter, the finished chunk one AllGather hop
    // later), and a workgroup-scope invalidate leaves the L1 copy in place.
    bool local = false;
    const uint64_t arrivals = a.sync == SYNC_BARRIER ? (uint64_t)(R - 1) : 1;
    const bool injected = r == 0 && lane == 0;

    // this workgroup's element range, relative to the start of any chunk
    const uint64_t off_lo = (uint64_t)j * a.slice_len + (uint64_t)w * a.sub_len;
    const uint64_t off_hi =
        umin(off_lo + a.sub_len, umin((uint64_t)(j + 1) * a.slice_len, a.chunk_len));

    for (int g = a.g_first; g <= a.g_last; ++g) {
        if (g > a.g_first) {
            if (threadIdx.x == 0) {
                uint64_t target = shadow + arrivals;
                if ((a.inject & RR_INJECT_EXTRA_EXPECTED) && injected && g == a.g_first + 1)
                    target += 1;
                const WaitResult res = sig_wait(&a.sig[(uint64_t)my_slot * kSignalStride], target,
                                                a.err, a.timeout_ticks);
                if (res.status == WAIT_TIMEOUT)
                    record_timeout(a.err, lane, r, g, target, res.observed);
                shadow = target;
                s_stop = res.status != WAIT_OK;
                // Acquire for the whole workgroup: drop this CU's L1 copies (and
                // non-coherent L2 lines), and finish that before any wave loads.
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            __syncthreads();
            if (s_stop) return;
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
        const uint64_t base = (uint64_t)c * a.chunk_len;
        const uint64_t lo = base + off_lo;
        const uint64_t hi = umin(base + off_hi, a.count);
        if (lo < hi) hop_body<DT, OP, BLOCK, U>(reduce, a.bufs[r], a.bufs[succ], lo, hi);

        if (g < a.g_last) {
            if (g == a.g_first) {
                if (threadIdx.x < 64) {
                    const int v = lane_on_one_xcd(a, lane, my_xcc);
                    if (threadIdx.x == 0) {
                        if (v < 0) record_timeout(a.err, lane, r, 0, a.generation, 0);
                        s_local = v;
                    }
                }
                __syncthreads();
                if (s_local < 0) return;
                local = s_local == 1;
            }
            if (local)
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // stores have reached L2
            else
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __syncthreads();
            const bool drop = (a.inject & RR_INJECT_DROP_ARRIVAL) && injected && g == a.g_first;
            if (!drop) {
                if (a.sync == SYNC_BARRIER) {
                    if ((int)threadIdx.x < R - 1) {
                        const int q = wrap(r + 1 + (int)threadIdx.x, R);
                        sig_add(&a.sig[(uint64_t)(lane * R + q) * kSignalStride], 1);
                    }
                } else if (threadIdx.x == 0) {
                    sig_add(&a.sig[(uint64_t)(lane * R + succ) * kSignalStride], 1);
                }
            }
        }
    }
    if (synced && threadIdx.x == 0) a.shadow[my_slot] = shadow;  // sig == shadow again
}

// ---------------------------------------------------------- barrier only --

struct BarrierArgs {
    uint64_t* sig;
    uint64_t* shadow;
    ErrorRecord* err;
    uint64_t timeout_ticks;
    uint64_t expected;  // arrivals per step
    int32_t R;          // waiters per context taking part
    int32_t stride;     // waiters per context in the object's layout
    int32_t nsteps;
    int32_t mode;       // SYNC_P2P or SYNC_BARRIER
    uint32_t inject;
    int32_t pad;
};

// One 64-lane workgroup per (context, waiter).  Each step: release, arrive,
// advance the shadow by `expected`, wait, acquire.
__global__ void __launch_bounds__(64) barrier_kernel(const BarrierArgs a) {
    const int ctx = blockIdx.x / a.R;
    const int r = blockIdx.x - ctx * a.R;
    const int slot = ctx * a.stride + r;
    if (a.nsteps <= 0) return;
    __shared__ int s_stop;
    uint64_t shadow = 0;
    if (threadIdx.x == 0) {
        s_stop = sig_read(&a.err->flag) != 0;
        shadow = a.shadow[slot];
    }
    __syncthreads();
    if (s_stop) return;
    const bool injected = r == 0 && ctx == 0;
    for (int step = 1; step <= a.nsteps; ++step) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const bool drop = (a.inject & RR_INJECT_DROP_ARRIVAL) && injected && step == 1;
        if (!drop) {
            if (a.mode == SYNC_BARRIER) {
                if ((int)threadIdx.x < a.R - 1) {
                    const int q = wrap(r + 1 + (int)threadIdx.x, a.R);
                    sig_add(&a.sig[(uint64_t)(ctx * a.stride + q) * kSignalStride], 1);
                }
            } else if (threadIdx.x == 0) {
                const int q = r + 1 == a.R ? 0 : r + 1;
                sig_add(&a.sig[(uint64_t)(ctx * a.stride + q) * kSignalStride], 1);
            }
        }
        if (threadIdx.x == 0) {
            uint64_t target = shadow + a.expected;
            if ((a.inject & RR_INJECT_EXTRA_EXPECTED) && injected && step == 1) target += 1;
            const WaitResult res = sig_wait(&a.sig[(uint64_t)slot * kSignalStride], target, a.err,
                                            a.timeout_ticks);
            if (res.status == WAIT_TIMEOUT) record_timeout(a.err, ctx, r, step, target, res.observed);
            shadow = target;
            s_stop = res.status != WAIT_OK;
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
        if (s_stop) return;
    }
    if (threadIdx.x == 0) a.shadow[slot] = shadow;
}

// ------------------------------------------------------ support kernels --

__global__ void __launch_bounds__(256) fill_u64_kernel(uint64_t* p, uint64_t n, uint64_t value,
                                                       uint64_t stride) {
    for (uint64_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += (uint64_t)gridDim.x * 256ull)
        p[i * stride] = value;
}

// Streaming copy: the bandwidth reference for the ring kernels.  Each
// workgroup copies one contiguous span (DRAM pages stay open longer than with a
// grid-wide stride); nontemporal hints, as the data are touched once.
__global__ void __launch_bounds__(256) copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, uint64_t nvec,
                                                   const uint8_t* __restrict__ src_tail,
                                                   uint8_t* __restrict__ dst_tail, uint32_t ntail) {
    constexpr int U = 8;
    const uint64_t per = (nvec + gridDim.x - 1) / gridDim.x;
    const uint64_t lo = (uint64_t)blockIdx.x * per;
    const uint64_t hi = lo + per < nvec ? lo + per : nvec;
    uint64_t i = lo + threadIdx.x;
    for (; i + (U - 1) * 256 < hi; i += U * 256) {
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(&src[i + u * 256]);
#pragma unroll
        for (int u = 0; u < U; ++u) __builtin_nontemporal_store(x[u], &dst[i + u * 256]);
    }
    for (; i < hi; i += 256) dst[i] = src[i];
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
    uint32_t generation = 0;
};

std::mutex g_mu;
DeviceState g_dev[kMaxDevices];

struct Plan {
    int sync;
    int team;
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

static size_t elem_bytes(int dt) { return dt == RR_BF16 ? 2 : 4; }

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
        // signals (one per cache line), shadows, the XCC table, the error record
        const size_t words = (size_t)kSlots * kSignalStride + 2 * (size_t)kSlots + 16;
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
        case 256: return ring_kernel<DT, OP, 256>;
        case 512: return ring_kernel<DT, OP, 512>;
        case 1024: return ring_kernel<DT, OP, 1024>;
        default: return nullptr;
    }
}

static RingKernel pick_ring_kernel(int dt, int op, int block) {
    if (dt == RR_INT32) return op == RR_SUM ? ring_kernel_for_block<DT_I32, OP_SUM>(block)
                                             : ring_kernel_for_block<DT_I32, OP_MAX>(block);
    if (dt == RR_FP32) return op == RR_SUM ? ring_kernel_for_block<DT_F32, OP_SUM>(block)
                                            : ring_kernel_for_block<DT_F32, OP_MAX>(block);
    return op == RR_SUM ? ring_kernel_for_block<DT_BF16, OP_SUM>(block)
                        : ring_kernel_for_block<DT_BF16, OP_MAX>(block);
}

// Argument checks that need no device.
static rr_status_t check_args(void* const* bufs, int R, size_t count, int dt, int op, int nslices,
                              const rr_options_t* opt) {
    if (R < 1 || R > RR_MAX_RANKS) return RR_ERR_INVALID;
    if (nslices < 1 || nslices > RR_MAX_SLICES) return RR_ERR_INVALID;
    if (dt != RR_INT32 && dt != RR_FP32 && dt != RR_BF16) return RR_ERR_INVALID;
    if (op != RR_SUM && op != RR_MAX) return RR_ERR_INVALID;
    if (count > (size_t)1 << 40) return RR_ERR_INVALID;
    if (opt) {
        if (opt->sync < RR_SYNC_AUTO || opt->sync > RR_SYNC_LAUNCH) return RR_ERR_INVALID;
        if (opt->team < 0 || opt->team > 4096) return RR_ERR_INVALID;
        if (opt->block != 0 && opt->block != 256 && opt->block != 512 && opt->block != 1024)
            return RR_ERR_INVALID;
    }
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
    const int block = opt && opt->block ? opt->block : 512;
    const int requested = opt ? opt->sync : RR_SYNC_AUTO;
    const uint32_t flags = opt ? opt->flags : 0;
    p->block = block;
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
    p->hbm_bytes = R > 1 ? rs + ag : 0;

    const void* kernel = (const void*)pick_ring_kernel(dt, op, block);
    p->resident_max = resident_limit(d, kernel, block);
    const int units = R * nslices;

    // team: about 16 waves per CU (two 512-thread workgroups), but each
    // workgroup keeps at least one full unrolled pass of work per hop.
    int team;
    if (opt && opt->team > 0) {
        team = opt->team;
    } else {
        const int target = d->cus * 16 * 64 / block;
        const uint64_t slice_vecs = p->slice_len / V;
        const uint64_t min_vecs = (uint64_t)block * 4;
        const uint64_t by_size = std::max<uint64_t>(1, slice_vecs / min_vecs);
        team = (int)std::min<uint64_t>(by_size, (uint64_t)std::max(1, target / units));
        team = std::max(team, 1);
    }
    // every lane needs R signals in the workspace
    const int max_team = std::max(1, kSlots / (R * nslices));
    if (team > max_team) {
        if (opt && opt->team > 0) return RR_ERR_UNSUPPORTED;
        team = max_team;
    }
    p->team = team;
    p->sub_len = round_up(ceil_div(p->slice_len, (uint64_t)team), V);
    p->grid = units * team;
    if ((long long)units * team > (1ll << 30)) return RR_ERR_INVALID;

    const bool multi_hop = p->g_last > p->g_first;
    int sync = requested;
    if (sync == RR_SYNC_AUTO) sync = multi_hop && p->grid <= p->resident_max ? RR_SYNC_P2P : RR_SYNC_LAUNCH;
    if ((sync == RR_SYNC_P2P || sync == RR_SYNC_BARRIER) && multi_hop && p->grid > p->resident_max)
        return RR_ERR_UNSUPPORTED;
    if (!multi_hop && sync != RR_SYNC_LAUNCH) sync = RR_SYNC_LAUNCH;  // one hop needs no hand-off
    p->sync = sync;
    p->launches = sync == RR_SYNC_LAUNCH ? p->g_last - p->g_first + 1 : 1;
    p->xcd_map = !(flags & RR_FLAG_NO_XCD_MAP) && (nslices * team) % 8 == 0 ? 1 : 0;
    p->coop = sync != RR_SYNC_LAUNCH && (flags & RR_FLAG_COOPERATIVE) ? 1 : 0;
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
    {
        std::lock_guard<std::mutex> lock(g_mu);
        if (++d->generation == 0) d->generation = 1;
        a.generation = d->generation;
    }
    a.R = R;
    a.team = p.team;
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
    uint64_t* mem;     // signals (stride kSignalStride), then shadows
    uint64_t* sig;
    uint64_t* shadow;
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

rr_status_t rr_plan_query(int R, size_t count, rr_dtype_t dt, int nslices, int phase,
                          const rr_options_t* opt, rr_plan_t* out) {
    if (!out || phase < 0 || phase > 2) return RR_ERR_INVALID;
    if (R < 1 || R > RR_MAX_RANKS || nslices < 1 || nslices > RR_MAX_SLICES) return RR_ERR_INVALID;
    if (dt != RR_INT32 && dt != RR_FP32 && dt != RR_BF16) return RR_ERR_INVALID;
    DeviceState* d = nullptr;
    rr_status_t st = ensure_device(&d);
    if (st != RR_OK) return st;
    Plan p;
    if ((st = make_plan(d, R, count, dt, RR_SUM, nslices, phase, opt, &p)) != RR_OK) return st;
    out->sync = p.sync;
    out->team = p.team;
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
    const size_t words = slots * kSignalStride + slots;
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
    b->mem = (uint64_t*)p;
    b->sig = b->mem;
    b->shadow = b->mem + slots * kSignalStride;
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

rr_status_t counting_barrier_run(rr_counting_barrier_t* b, int R, int nsteps, int ncontexts,
                                 uint64_t expected_per_step, const rr_options_t* opt,
                                 rr_stream_t stream) {
    if (!b || R < 1 || R > b->nwaiters || ncontexts < 1 || ncontexts > b->ncontexts || nsteps < 0)
        return RR_ERR_INVALID;
    if (opt && (opt->sync < RR_SYNC_AUTO || opt->sync > RR_SYNC_LAUNCH)) return RR_ERR_INVALID;
    DeviceState* d = nullptr;
    rr_status_t st = ensure_device(&d);
    if (st != RR_OK) return st;
    const int grid = R * ncontexts;
    if (grid > resident_limit(d, (const void*)barrier_kernel, 64)) return RR_ERR_UNSUPPORTED;
    BarrierArgs a;
    memset(&a, 0, sizeof a);
    a.sig = b->sig;
    a.shadow = b->shadow;
    a.err = d->err;
    a.timeout_ticks = timeout_ticks(d, opt);
    a.expected = expected_per_step;
    a.R = R;
    a.stride = b->nwaiters;
    a.nsteps = nsteps;
    a.mode = opt && opt->sync == RR_SYNC_P2P ? SYNC_P2P : SYNC_BARRIER;
    a.inject = opt ? opt->inject : 0;
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
        rec->expected = e.expected;
        rec->observed = e.observed;
    }
    // clear the record and restore sig == shadow everywhere
    if ((st = fill(d->sig, kSlots, 0, kSignalStride, s)) != RR_OK) return st;
    if ((st = fill(d->shadow, kSlots, 0, 1, s)) != RR_OK) return st;
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
    return fill(d->shadow, kSlots, value, 1, s);
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
        1, std::min<uint64_t>((uint64_t)d->cus * 16, ceil_div(nvec, 2048)));
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
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
        (void)hipSetDevice(prev);
        d = DeviceState();
    }
}

}  // extern "C"
