// rr_ring_kernel.hpp -- the in-place ring kernel (ReduceScatter, AllGather and
// the AllReduce that chains them) over virtual ranks on one MI355X.  Included by
// one translation unit per element type (rr_ring_<type>.hip), which compile in
// parallel: each holds the 32 kernels of its type (4 reductions x 4 workgroup
// sizes x hop order).
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
// consumer advances its shadow by 1 and waits (P2P).  For a per-hop barrier (the
// counting barrier of the DeepEP pull request "make the rail barrier a counting
// barrier", section "Fix") every workgroup of the lane adds 1 to the lane's one
// shared signal and waits for it to advance by R, its own arrival included; or,
// with one signal per waiter, adds 1 to the R-1 other ranks' signals and waits
// for R-1 on its own.  A
// workgroup serves `depth` lanes interleaved hop by hop (one lane's hand-off
// completes while the other's hop runs) and `rounds` groups of lanes one after
// another (so that the lanes in flight keep a hop's partials cached until the
// next hop reads them).
//
// One producer per rank per signal is what makes the count safe to hand data
// over.  Had the W workgroups of a slice shared one signal, a workgroup running
// a hop ahead could supply the increment of a teammate that has not finished --
// the hazard the same pull request describes for anonymous counting (section
// "Scoped to the rail team": a count says that enough arrived, not who) -- and
// the consumer of that teammate's sub-range would read stale data.
#pragma once

#include "rr_kernels.hpp"

namespace rr {

// One hop of one workgroup over elements [lo, hi) of both buffers.  ReduceScatter:
// dst = fold(src, dst).  AllGather: dst = src, bit for bit.  16-byte vectors,
// U vectors per thread in flight, then a scalar tail (only at the ragged end).
// DESC runs the vectors from the top down.  The ring alternates (even hops top
// down) once its buffers outgrow the caches: what a hop reads from its
// predecessor's buffer was written one hop earlier in the opposite order, so
// the lines written last -- the likeliest to be still in the Infinity Cache --
// are read first, instead of every line waiting a whole hop.  Only the kernels
// instantiated with ALT carry the descending loops: the extra code made every
// hop of the latency-bound calls (which never alternate) 0.2-0.5 us slower.
template <int DT, int OP, int BLOCK, int U, int AUX, bool DESC>
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
    // descending: vector k of the pass order is vector nv - 1 - k
    const uint32_t top = nv - 1;
#define RR_AT(k) (DESC ? top - (uint32_t)(k) : (uint32_t)(k))
    uint32_t i = threadIdx.x;
    if (reduce && d2) {
        // recvReduceCopySend: the finished chunk goes to the owner's buffer and on
        // to the owner's successor in the same pass
        for (; i + (U - 1) * BLOCK < nv; i += U * BLOCK) {
            u32x4 x[U], y[U];
#pragma unroll
            for (int u = 0; u < U; ++u) x[u] = load_in<AUX>(rs, RR_AT(i + u * BLOCK));
#pragma unroll
            for (int u = 0; u < U; ++u) y[u] = d[RR_AT(i + u * BLOCK)];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const u32x4 v = fold4<DT, OP>(x[u], y[u]);
                d[RR_AT(i + u * BLOCK)] = v;
                d2[RR_AT(i + u * BLOCK)] = v;
            }
        }
        for (; i < nv; i += BLOCK) {
            const u32x4 v = fold4<DT, OP>(load_in<AUX>(rs, RR_AT(i)), d[RR_AT(i)]);
            d[RR_AT(i)] = v;
            d2[RR_AT(i)] = v;
        }
    } else if (reduce) {
        for (; i + (U - 1) * BLOCK < nv; i += U * BLOCK) {
            u32x4 x[U], y[U];
#pragma unroll
            for (int u = 0; u < U; ++u) x[u] = load_in<AUX>(rs, RR_AT(i + u * BLOCK));
#pragma unroll
            for (int u = 0; u < U; ++u) y[u] = d[RR_AT(i + u * BLOCK)];
#pragma unroll
            for (int u = 0; u < U; ++u) d[RR_AT(i + u * BLOCK)] = fold4<DT, OP>(x[u], y[u]);
        }
        for (; i < nv; i += BLOCK) d[RR_AT(i)] = fold4<DT, OP>(load_in<AUX>(rs, RR_AT(i)), d[RR_AT(i)]);
    } else {
        constexpr int UC = 2 * U;
        for (; i + (UC - 1) * BLOCK < nv; i += UC * BLOCK) {
            u32x4 x[UC];
#pragma unroll
            for (int u = 0; u < UC; ++u) x[u] = load_in<AUX>(rs, RR_AT(i + u * BLOCK));
#pragma unroll
            for (int u = 0; u < UC; ++u) d[RR_AT(i + u * BLOCK)] = x[u];
        }
        for (; i < nv; i += BLOCK) d[RR_AT(i)] = load_in<AUX>(rs, RR_AT(i));
    }
#undef RR_AT
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

template <int DT, int OP, int BLOCK, int U, bool ALT>
__device__ __forceinline__ void hop_body(bool reduce, bool stream, const void* srcbuf,
                                         void* dstbuf, void* dst2buf, uint64_t lo, uint64_t hi,
                                         bool desc) {
    constexpr uint64_t kPiece = kPieceBytes / ElemBytes<DT>::value;  // elements, vector multiple
    for (uint64_t p = lo; p < hi; p += kPiece) {
        const uint64_t q = umin(p + kPiece, hi);
        if constexpr (ALT) {
            if (stream && desc)
                hop_piece<DT, OP, BLOCK, U, kAuxRingIncoming, true>(reduce, srcbuf, dstbuf, dst2buf,
                                                                     p, q);
            else if (stream)
                hop_piece<DT, OP, BLOCK, U, kAuxRingIncoming, false>(reduce, srcbuf, dstbuf,
                                                                      dst2buf, p, q);
            else if (desc)
                hop_piece<DT, OP, BLOCK, U, kAuxDeviceScope, true>(reduce, srcbuf, dstbuf, dst2buf,
                                                                    p, q);
            else
                hop_piece<DT, OP, BLOCK, U, kAuxDeviceScope, false>(reduce, srcbuf, dstbuf,
                                                                     dst2buf, p, q);
        } else if (stream) {
            hop_piece<DT, OP, BLOCK, U, kAuxRingIncoming, false>(reduce, srcbuf, dstbuf, dst2buf,
                                                                  p, q);
        } else {
            hop_piece<DT, OP, BLOCK, U, kAuxDeviceScope, false>(reduce, srcbuf, dstbuf, dst2buf, p,
                                                                 q);
        }
    }
}

template <int DT, int OP, int BLOCK, bool ALT>
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
    // Arrivals a waiter expects per hop: its predecessor's (P2P); the R-1 other
    // ranks' (barrier, a signal per waiter); all R ranks' (barrier, one signal
    // per lane that every rank of the lane adds to, its own arrival included).
    const bool shared = a.sync == SYNC_BARRIER && a.shared_sig != 0;
    const uint64_t arrivals =
        a.sync == SYNC_BARRIER ? (uint64_t)(shared ? R : R - 1) : 1;
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
            if (p < a.depth && synced && threadIdx.x == 0)
                shadow[p] = shared ? a.lane_shadow[lane[p]] : a.shadow[lane[p] * R + r];
        }

        for (int g = a.g_first; g <= a.g_last; ++g) {
#pragma unroll
            for (int p = 0; p < kMaxDepth; ++p) {
                if (p >= a.depth) break;
                const int my_slot = lane[p] * R + r;
                const bool injected = r == 0 && lane[p] == 0;
                uint64_t t_wait = 0, t_hop = 0;
                if (a.stamps && threadIdx.x == 0) t_wait = wall_clock64();
                if (g > a.g_first) {
                    if (threadIdx.x == 0) {
                        uint64_t target = shadow[p] + arrivals;
                        if ((a.inject & RR_INJECT_EXTRA_EXPECTED) && injected &&
                            g == a.g_first + 1)
                            target += 1;
                        const uint64_t* wsig =
                            shared ? &a.lane_sig[(uint64_t)lane[p] * kSignalStride]
                                   : &a.sig[(uint64_t)my_slot * kSignalStride];
                        const WaitResult res =
                            sig_wait(wsig, target, a.err, a.timeout_ticks, a.nap);
                        if (res.status == WAIT_TIMEOUT)
                            record_timeout(a.err, lane[p], r, g, target, res.observed);
                        shadow[p] = target;
                        s_stop_lane[p] = res.status != WAIT_OK;
                        acquire_stores(local);
                    }
                    __syncthreads();
                    if (s_stop_lane[p]) return;
                }
                if (a.stamps && threadIdx.x == 0) t_hop = wall_clock64();

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
                    hop_body<DT, OP, BLOCK, U, ALT>(reduce, a.stream_in != 0, a.bufs[r],
                                                    a.bufs[succ], dst2, lo, hi, (g & 1) == 0);

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
                        if (shared) {
                            if (threadIdx.x == 0)
                                sig_add(&a.lane_sig[(uint64_t)lane[p] * kSignalStride], 1);
                        } else if (a.sync == SYNC_BARRIER) {
                            if ((int)threadIdx.x < R - 1) {
                                const int q = wrap(r + 1 + (int)threadIdx.x, R);
                                sig_add(&a.sig[(uint64_t)(lane[p] * R + q) * kSignalStride], 1);
                            }
                        } else if (threadIdx.x == 0) {
                            sig_add(&a.sig[(uint64_t)(lane[p] * R + succ) * kSignalStride], 1);
                        }
                    }
                }
                if (a.stamps && threadIdx.x == 0) {
                    uint64_t* st = a.stamps +
                                   ((uint64_t)my_slot * (2 * (R - 1)) + (uint64_t)(g - 1)) * 3;
                    st[0] = t_wait;
                    st[1] = t_hop;
                    st[2] = wall_clock64();
                }
            }
        }
        if (synced && threadIdx.x == 0) {
#pragma unroll
            for (int p = 0; p < kMaxDepth; ++p)
                if (p < a.depth) {  // signal == shadow again
                    if (shared)
                        a.lane_shadow[lane[p]] = shadow[p];  // every rank stores the same value
                    else
                        a.shadow[lane[p] * R + r] = shadow[p];
                }
        }
    }
}

// At least four waves per SIMD (two 512-thread or one 1024-thread workgroup per
// CU, which every plan needs): the 16-bit kernels otherwise take more registers.
// ALT: the even hops run top down.
template <int DT, int OP, int BLOCK, bool ALT>
__global__ void __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4)))
ring_kernel(const RingArgs a) {
    ring_body<DT, OP, BLOCK, ALT>(a, launch_generation(a.launch));
    leave_launch(a.launch);
}

template <int DT, int OP, bool ALT>
static RingKernel ring_kernel_for_block(int block) {
    switch (block) {
        case 128: return ring_kernel<DT, OP, 128, ALT>;
        case 256: return ring_kernel<DT, OP, 256, ALT>;
        case 512: return ring_kernel<DT, OP, 512, ALT>;
        case 1024: return ring_kernel<DT, OP, 1024, ALT>;
        default: return nullptr;
    }
}

template <int DT, bool ALT>
static RingKernel ring_kernel_for_op(int op, int block) {
    switch (op) {
        case RR_SUM: return ring_kernel_for_block<DT, OP_SUM, ALT>(block);
        case RR_MAX: return ring_kernel_for_block<DT, OP_MAX, ALT>(block);
        case RR_MIN: return ring_kernel_for_block<DT, OP_MIN, ALT>(block);
        case RR_PROD: return ring_kernel_for_block<DT, OP_PROD, ALT>(block);
        default: return nullptr;
    }
}

// The kernel for (op, block, hop order) of element type DT.
template <int DT>
RingKernel ring_kernel_for_type(int op, int block, bool alternate) {
    return alternate ? ring_kernel_for_op<DT, true>(op, block)
                     : ring_kernel_for_op<DT, false>(op, block);
}

}  // namespace rr
