// rr_device.hpp -- device-side building blocks of the ring kernels (gfx950).
//
//  * element folds for int32 / fp32 / bf16 / fp16, SUM, MAX, MIN and PROD, on
//    16-byte vectors;
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

enum : int { DT_I32 = 0, DT_F32 = 1, DT_BF16 = 2, DT_F16 = 3 };
enum : int { OP_SUM = 0, OP_MAX = 1, OP_MIN = 2, OP_PROD = 3 };
enum : int { SYNC_NONE = 0, SYNC_P2P = 1, SYNC_BARRIER = 2, SYNC_PER_PEER = 3 };

template <int DT> struct ElemBytes {
    static constexpr int value = DT == DT_BF16 || DT == DT_F16 ? 2 : 4;
};

// ------------------------------------------------------------------ folds --
// fold(in, local): the receiver's new value, `in` being the incoming partial.
// SUM and PROD: one operation, rounded to the storage format (int32 wraps).
// MAX (MIN): the local value if it compares greater (less), else the incoming
// one -- a selection, no arithmetic.

// Round a binary32 value to the nearest bfloat16, ties to even; any NaN becomes
// the quiet NaN 0x7FC0.  Adding 0x7FFF plus the lowest kept bit and truncating
// rounds the 16 dropped bits to nearest, ties to even; a carry out of the
// significand moves to the exponent, so the largest values round to infinity.
__device__ __forceinline__ uint32_t bf16_round(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return (u & 0x7FFFFFFFu) > 0x7F800000u ? 0x7FC0u : r;
}

// The 16-bit formats, two to a 32-bit lane (the lower address in the low half).
// A bf16 or fp16 SUM or PROD is computed in binary32 and rounded once to the
// format: equal to the correctly rounded operation, because binary32 holds the
// exact product of two such values (fp16) or enough of it that no false tie
// arises (bf16: at most 16 significant bits), and because 24 >= 2p + 2 for the
// sums (p = 8, 11).
template <int DT> struct Codec;
template <> struct Codec<DT_BF16> {
    __device__ static float lo(uint32_t p) { return __uint_as_float(p << 16); }
    __device__ static float hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }
    __device__ static uint32_t round(float f) { return bf16_round(f); }
};
template <> struct Codec<DT_F16> {
    __device__ static float lo(uint32_t p) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xFFFFu));
    }
    __device__ static float hi(uint32_t p) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(p >> 16));
    }
    // round to nearest even (the default mode of the conversion); NaN -> 0x7E00.
    // The empty asm keeps the binary32 result as it is: without it the compiler
    // folds "multiply, then convert" into one mixed-precision fma with a +0
    // addend, which turns a -0 product into +0.
    __device__ static uint32_t round(float f) {
        asm volatile("" : "+v"(f));
        return f != f ? 0x7E00u : (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
    }
};

template <int OP> __device__ __forceinline__ float arith(float in, float lo) {
    return OP == OP_PROD ? in * lo : in + lo;
}
template <int OP, typename T> __device__ __forceinline__ bool local_wins(T in, T lo) {
    return OP == OP_MAX ? lo > in : lo < in;
}

template <int DT, int OP> struct Fold {
    static constexpr bool kArith = OP == OP_SUM || OP == OP_PROD;

    // One 16-bit element, operands in the low 16 bits.
    __device__ static uint32_t half(uint32_t in, uint32_t lo) {
        const float a = Codec<DT>::lo(in), b = Codec<DT>::lo(lo);
        if constexpr (kArith) return Codec<DT>::round(arith<OP>(a, b));
        return local_wins<OP>(a, b) ? (lo & 0xFFFFu) : (in & 0xFFFFu);
    }

    // One 32-bit lane: one int32 / fp32 element or two 16-bit elements.
    __device__ static uint32_t lane(uint32_t in, uint32_t lo) {
        if constexpr (DT == DT_I32) {
            if constexpr (OP == OP_SUM) return in + lo;   // wraps
            if constexpr (OP == OP_PROD) return in * lo;  // low 32 bits: wraps
            return local_wins<OP>((int32_t)in, (int32_t)lo) ? lo : in;
        } else if constexpr (DT == DT_F32) {
            const float a = __uint_as_float(in), b = __uint_as_float(lo);
            if constexpr (kArith) return __float_as_uint(arith<OP>(a, b));
            return local_wins<OP>(a, b) ? lo : in;
        } else {
            const float al = Codec<DT>::lo(in), bl = Codec<DT>::lo(lo);
            const float ah = Codec<DT>::hi(in), bh = Codec<DT>::hi(lo);
            if constexpr (kArith) {
                return Codec<DT>::round(arith<OP>(al, bl)) |
                       (Codec<DT>::round(arith<OP>(ah, bh)) << 16);
            }
            const uint32_t l = local_wins<OP>(al, bl) ? lo : in;
            const uint32_t h = local_wins<OP>(ah, bh) ? lo : in;
            return (l & 0xFFFFu) | (h & 0xFFFF0000u);
        }
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
    if constexpr (ElemBytes<DT>::value == 2) {
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
// nap: how long to sleep between polls -- 0: 64 clocks, 1: 512, 2: 4096.  A
// counting barrier's signal takes R-1 atomic adds per step; frequent polls of
// the same line slow them and the data traffic around them, which costs more
// than the later wake-up once a hop moves enough data (the R=64 ring: +2%).
__device__ __forceinline__ WaitResult sig_wait(const uint64_t* sig, uint64_t target,
                                               const ErrorRecord* err, uint64_t timeout_ticks,
                                               int nap = 0) {
    uint64_t v = sig_read(sig);
    if (rolling_le(target, v)) return {WAIT_OK, v};
    const uint64_t start = wall_clock64();
    uint32_t spins = 0;
    for (;;) {
        if (nap >= 2)
            __builtin_amdgcn_s_sleep(64);
        else if (nap == 1)
            __builtin_amdgcn_s_sleep(8);
        else
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
