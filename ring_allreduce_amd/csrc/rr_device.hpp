// rr_device.hpp -- device-side building blocks of the ring kernels (gfx950).
//
//  * element folds for int32 / fp32 / bf16, SUM and MAX, on 16-byte vectors;
//  * the counting-signal layer: 64-bit agent-scope counters in HBM, waiters
//    holding a private shadow, rolling comparison, bounded waits.
//
// The signal idiom follows two pages: the 2kiu.com article on NCCL GIN (section
// "Signals and counters": 64-bit signals with a rolling comparison that keeps
// x < x + 1 across wrap, and per-signal shadows), and the DeepEP pull request
// "make the rail barrier a counting barrier" (section "Fix": every peer adds 1
// to one signal and the waiter advances its shadow by the number of arrivals it
// expects).  On one device, agent-scope release (producer) and acquire
// (consumer) make every hop's stores visible to the next hop's loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum : int { DT_I32 = 0, DT_F32 = 1, DT_BF16 = 2 };
enum : int { OP_SUM = 0, OP_MAX = 1 };
enum : int { SYNC_NONE = 0, SYNC_P2P = 1, SYNC_BARRIER = 2, SYNC_PER_PEER = 3 };

template <int DT> struct ElemBytes { static constexpr int value = DT == DT_BF16 ? 2 : 4; };

// ------------------------------------------------------------------ folds --
// fold(in, local): the receiver's new value, `in` being the incoming partial.

// Round a binary32 value to the nearest bfloat16, ties to even; any NaN becomes
// the quiet NaN 0x7FC0.  Adding 0x7FFF plus the lowest kept bit and truncating
// rounds the 16 dropped bits to nearest, ties to even; a carry out of the
// significand moves to the exponent, so the largest values round to infinity.
__device__ __forceinline__ uint32_t bf16_round(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return (u & 0x7FFFFFFFu) > 0x7F800000u ? 0x7FC0u : r;
}

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

template <int DT, int OP> struct Fold;

template <> struct Fold<DT_I32, OP_SUM> {
    __device__ static uint32_t lane(uint32_t in, uint32_t lo) { return in + lo; }  // wraps
};
template <> struct Fold<DT_I32, OP_MAX> {
    __device__ static uint32_t lane(uint32_t in, uint32_t lo) {
        return (int32_t)lo > (int32_t)in ? lo : in;
    }
};
template <> struct Fold<DT_F32, OP_SUM> {
    __device__ static uint32_t lane(uint32_t in, uint32_t lo) {
        return __float_as_uint(__uint_as_float(in) + __uint_as_float(lo));
    }
};
template <> struct Fold<DT_F32, OP_MAX> {
    __device__ static uint32_t lane(uint32_t in, uint32_t lo) {
        return __uint_as_float(lo) > __uint_as_float(in) ? lo : in;
    }
};
// bf16: a 32-bit lane carries two elements, the lower address in the low half.
template <> struct Fold<DT_BF16, OP_SUM> {
    __device__ static uint32_t half(uint32_t in, uint32_t lo) {  // operands in the low 16 bits
        return bf16_round(bf16_lo(in) + bf16_lo(lo));
    }
    __device__ static uint32_t lane(uint32_t in, uint32_t lo) {
        const uint32_t a = bf16_round(bf16_lo(in) + bf16_lo(lo));
        const uint32_t b = bf16_round(bf16_hi(in) + bf16_hi(lo));
        return a | (b << 16);
    }
};
template <> struct Fold<DT_BF16, OP_MAX> {
    __device__ static uint32_t half(uint32_t in, uint32_t lo) {
        return bf16_lo(lo) > bf16_lo(in) ? (lo & 0xFFFFu) : (in & 0xFFFFu);
    }
    __device__ static uint32_t lane(uint32_t in, uint32_t lo) {
        const uint32_t a = bf16_lo(lo) > bf16_lo(in) ? lo : in;
        const uint32_t b = bf16_hi(lo) > bf16_hi(in) ? lo : in;
        return (a & 0xFFFFu) | (b & 0xFFFF0000u);
    }
};

template <int DT, int OP>
__device__ __forceinline__ u32x4 fold4(u32x4 in, u32x4 lo) {
    u32x4 r;
    r.x = Fold<DT, OP>::lane(in.x, lo.x);
    r.y = Fold<DT, OP>::lane(in.y, lo.y);
    r.z = Fold<DT, OP>::lane(in.z, lo.z);
    r.w = Fold<DT, OP>::lane(in.w, lo.w);
    return r;
}

// One element at a time, for the ragged end of the last chunk.
template <int DT, int OP>
__device__ __forceinline__ void fold_one(const void* in, void* lo) {
    if constexpr (DT == DT_BF16) {
        const uint16_t a = *(const uint16_t*)in;
        uint16_t* b = (uint16_t*)lo;
        *b = (uint16_t)Fold<DT, OP>::half(a, *b);
    } else {
        const uint32_t a = *(const uint32_t*)in;
        uint32_t* b = (uint32_t*)lo;
        *b = Fold<DT, OP>::lane(a, *b);
    }
}

// --------------------------------------------------------- signal layer --

// One signal per cache line, so pollers of one signal do not share a line with
// producers of another.
constexpr int kSignalStride = 16;  // uint64 words = 128 bytes

// Device failure record; layout shared with the host side of this library.
struct ErrorRecord {
    uint64_t flag;      // 0 = clear; set once by the first waiter that gives up
    int32_t status;
    int32_t ctx;
    int32_t waiter;
    int32_t hop;
    int32_t peer;       // the peer whose arrival is missing; -1 for a counting signal
    int32_t pad;
    uint64_t expected;
    uint64_t observed;
};

// a <= b in the rolling (serial-number) order of 64-bit counters: true when b
// is at most 2^63 - 1 steps ahead of a, so x <= x + 1 holds across the wrap.
__device__ __forceinline__ bool rolling_le(uint64_t a, uint64_t b) {
    return (int64_t)(b - a) >= 0;
}

__device__ __forceinline__ uint64_t sig_read(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void sig_add(uint64_t* p, uint64_t n) {
    __hip_atomic_fetch_add(p, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

enum : int { WAIT_OK = 0, WAIT_TIMEOUT = 1, WAIT_ABORT = 2 };

struct WaitResult {
    int status;         // WAIT_*
    uint64_t observed;  // last value read
};

// Called by one lane.  Returns once rolling_le(target, *sig); gives up after
// `timeout_ticks` of the constant-rate wall clock, or as soon as another
// waiter on the device has given up (err->flag set).
__device__ __forceinline__ WaitResult sig_wait(const uint64_t* sig, uint64_t target,
                                               const ErrorRecord* err, uint64_t timeout_ticks) {
    uint64_t v = sig_read(sig);
    if (rolling_le(target, v)) return {WAIT_OK, v};
    const uint64_t start = wall_clock64();
    uint32_t spins = 0;
    for (;;) {
        __builtin_amdgcn_s_sleep(1);
        v = sig_read(sig);
        if (rolling_le(target, v)) return {WAIT_OK, v};
        if ((++spins & 31u) == 0u) {
            if (sig_read(&err->flag) != 0) return {WAIT_ABORT, v};
            if (wall_clock64() - start > timeout_ticks) return {WAIT_TIMEOUT, v};
        }
    }
}

// First give-up on the device wins the record; later ones only stop.
__device__ __noinline__ void record_timeout(ErrorRecord* err, int ctx, int waiter, int hop,
                                            uint64_t expected, uint64_t observed, int peer = -1) {
    uint64_t clear = 0;
    if (__hip_atomic_compare_exchange_strong(&err->flag, &clear, (uint64_t)1, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        err->status = 4;  // RR_ERR_TIMEOUT
        err->ctx = ctx;
        err->waiter = waiter;
        err->hop = hop;
        err->peer = peer;
        err->expected = expected;
        err->observed = observed;
    }
}

}  // namespace rr
