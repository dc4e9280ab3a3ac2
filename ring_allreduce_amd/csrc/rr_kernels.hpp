// rr_kernels.hpp -- what the kernel families of the library and its host side
// share: sizes fixed at compile time, the launch arguments of every kernel, the
// device helpers the kernels have in common (the per-launch tag, the XCD-aware
// block map, the hand-off fences, bounded loads of incoming data), and the typed
// kernel pointers the host side launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr.h"
#include "rr_device.hpp"

namespace rr {

constexpr int kMaxDevices = 64;
constexpr int kMaxDepth = 4;
constexpr int kSlots = RR_MAX_SLICES * RR_MAX_RANKS;  // (context, rank) pairs

// Per-launch tag of the XCD table, kept on the device so that a launch replayed
// from a captured graph still gets a fresh one: every workgroup reads `gen` at
// start, and the last workgroup to leave a launch advances it for the next
// launch (launches on one device are ordered, so no launch starts before the
// previous one has left).  Table entries carry a published bit, so a zeroed
// table matches no tag, and zeroed memory (tag, exit count, table) is a valid
// starting state.
struct LaunchTag {
    uint64_t* gen;    // current tag (its low 32 bits)
    uint64_t* exits;  // workgroups of the running launch that have left
};

// The in-place ring (one launch runs hops g_first..g_last).
struct RingArgs {
    void* bufs[RR_MAX_RANKS];
    uint64_t count;      // elements per rank
    uint64_t chunk_len;  // nominal chunk length (elements, vector multiple)
    uint64_t slice_len;  // nominal slice length
    uint64_t sub_len;    // nominal length per team member
    uint64_t* sig;       // signal of slot s at sig[s * kSignalStride]
    uint64_t* shadow;    // shadow of slot s
    uint64_t* xcc_table; // per workgroup: (generation << 8) | published | XCC id, set at start
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
    int32_t nap;         // sleep between polls of a wait: 0 short, 1 medium, 2 long
    int32_t stream_in;   // loads of the predecessor's buffer are non-temporal
    int32_t shared_sig;  // barrier: one signal per lane that all R ranks add to (else
                         // one per waiter that the R-1 others add to)
    int32_t pad;
    uint64_t* lane_sig;    // shared_sig: signal of lane l at lane_sig[l * kSignalStride]
    uint64_t* lane_shadow; // shared_sig: the lane's shadow (every rank's waiter tracks it)
    uint64_t* stamps;      // optional: wall clock per (lane, rank, hop): wait begins, hop
                           // begins, hop ends (after its arrival); 3 words each
};

// The staged loop: receive slots per (lane, rank), threads per workgroup.
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
// What a staged launch computes.
enum : int { MODE_ALLREDUCE = 0, MODE_RS = 1, MODE_AG = 2 };

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

// The AlltoAll: one counting signal per receiver.
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

// The barrier alone (latency measurements and failure tests).
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
    int32_t shared;      // counting mode: one signal per context that every waiter adds to
    uint64_t* ctx_sig;   // shared: the context's signal at ctx_sig[ctx * kSignalStride]
    uint64_t* ctx_shadow;// shared: the context's shadow (every waiter tracks it)
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

// Workgroups are dealt to the 8 XCDs round-robin by index.  The ring, staged and
// barrier kernels lay their grid out as columns of R workgroups (one per rank)
// with every column on one XCD: block b = ((col / 8) * R + rank) * 8 + col % 8.
// Column counts are padded to a multiple of 8; padding columns exit at once.
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

// Every synchronising workgroup publishes (generation << 8) | published | XCC id
// at start.
constexpr uint64_t kXccPublished = 0x80;
__device__ __forceinline__ void publish_xcc(uint64_t* table, uint32_t generation, uint32_t xcc) {
    __hip_atomic_store(&table[blockIdx.x], ((uint64_t)generation << 8) | kXccPublished | xcc,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by wave 0.  1 when the R workgroups of column `col` all run on this
// workgroup's XCD (read from the published table), 0 if not; they then share one
// L2, the point where producer stores and consumer loads meet.  All R
// workgroups of the column compute the same answer.  -1 if one never published
// (timeout, or a failure elsewhere).
__device__ inline int column_on_one_xcd(const uint64_t* table, uint32_t generation, int R, int col,
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
        while ((uint32_t)(v >> 8) != generation || !(v & kXccPublished)) {
            __builtin_amdgcn_s_sleep(1);
            v = sig_read(e);
            if ((++spins & 31u) == 0u &&
                (sig_read(&err->flag) != 0 || wall_clock64() - start > timeout_ticks)) {
                failed = 1;
                break;
            }
        }
        same = !failed && (uint32_t)(v & 0x7Fu) == mine;
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

// ------------------------------------------------------ kernel pointers --
// Each kernel family is its own translation unit; these return the launchable
// kernel for a configuration, or nullptr when none is compiled for it.
typedef void (*RingKernel)(RingArgs);
typedef void (*StagedKernel)(StagedArgs);
typedef void (*AlltoallKernel)(A2AArgs);
typedef void (*BarrierKernel)(BarrierArgs);
typedef void (*FillKernel)(uint64_t*, uint64_t, uint64_t, uint64_t);
typedef void (*CopyKernel)(const u32x4*, u32x4*, uint64_t, const uint8_t*, uint8_t*, uint32_t);

// block 128, 256, 512 or 1024; alternate: the kernel whose even hops run top down.
// One translation unit per element type holds the ring kernels (rr_ring_<type>.hip).
RingKernel pick_ring_kernel_i32(int op, int block, bool alternate);
RingKernel pick_ring_kernel_f32(int op, int block, bool alternate);
RingKernel pick_ring_kernel_bf16(int op, int block, bool alternate);
RingKernel pick_ring_kernel_f16(int op, int block, bool alternate);
inline RingKernel pick_ring_kernel(int dt, int op, int block, bool alternate) {
    switch (dt) {
        case RR_INT32: return pick_ring_kernel_i32(op, block, alternate);
        case RR_FP32: return pick_ring_kernel_f32(op, block, alternate);
        case RR_BF16: return pick_ring_kernel_bf16(op, block, alternate);
        case RR_FP16: return pick_ring_kernel_f16(op, block, alternate);
        default: return nullptr;
    }
}
StagedKernel pick_staged_kernel(int dt, int op);
AlltoallKernel pick_alltoall_kernel(int elem_bytes);     // 2 or 4
BarrierKernel barrier_kernel_handle();
FillKernel fill_kernel_handle();
CopyKernel copy_kernel_handle();

}  // namespace rr
