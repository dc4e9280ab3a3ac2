// rr_aux_kernels.hip -- the AlltoAll, the barrier alone, and the support kernels
// (a 64-bit fill and the streaming copy that serves as the bandwidth reference).
#include "rr_kernels.hpp"

namespace rr {

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
//             expects R-1 on its own (the DeepEP pull request's counting barrier);
//             shared: one add to the context's one signal, which every waiter
//             of the context polls, expecting R (its own arrival included)
//   PER_PEER  one add to this waiter's slot in each other waiter's row; the
//             waiter expects every slot of its row to advance (the per-peer
//             layout the pull request replaced)
__device__ __forceinline__ void barrier_body(const BarrierArgs& a, const uint32_t generation) {
    const Place pl = place_of(blockIdx.x, a.R, true);
    const int r = pl.rank, ctx = pl.col;
    if (ctx >= a.nctx || a.nsteps <= 0) return;
    const int slot = ctx * a.stride + r;
    const bool shared = a.shared && a.mode == SYNC_BARRIER;
    uint64_t* const wait_sig =
        shared ? &a.ctx_sig[(uint64_t)ctx * kSignalStride] : &a.sig[(uint64_t)slot * kSignalStride];
    const uint32_t my_xcc = xcc_id() & 0xFu;
    __shared__ int s_stop;
    uint64_t shadow = 0;
    if (threadIdx.x == 0) {
        s_stop = sig_read(&a.err->flag) != 0;
        shadow = shared ? a.ctx_shadow[ctx] : a.shadow[slot];
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
    const bool audit = a.audit && a.mode == SYNC_BARRIER && !shared;
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
    const bool defer =
        (a.inject & RR_INJECT_DEFER_ARRIVAL) && injected && peer_lane && q == 1 && !shared;
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
            } else if (shared) {
                if (lane == 0) sig_add(wait_sig, 1);
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
                const WaitResult res = sig_wait(wait_sig, target, a.err, a.timeout_ticks);
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
        if (shared)
            a.ctx_shadow[ctx] = shadow;  // every waiter of the context stores the same value
        else if (!per_peer)
            a.shadow[slot] = shadow;
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

// ------------------------------------------------------ kernel pointers --

AlltoallKernel pick_alltoall_kernel(int elem_bytes) {
    switch (elem_bytes) {
        case 2: return alltoall_kernel<2, kA2ABlock>;
        case 4: return alltoall_kernel<4, kA2ABlock>;
        default: return nullptr;
    }
}

BarrierKernel barrier_kernel_handle() { return barrier_kernel; }
FillKernel fill_kernel_handle() { return fill_u64_kernel; }
CopyKernel copy_kernel_handle() { return copy_kernel; }

}  // namespace rr
