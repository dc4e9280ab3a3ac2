// rr_staged_kernel.hip -- the staged loop: the ring as the primitives of one
// rank, out of place, with receive slots and credits.
#include "rr_kernels.hpp"

namespace rr {

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

enum : int { P_SEND = 0, P_RRS = 1, P_RRCS = 2, P_RCS = 3, P_RECV = 4, P_RRC = 5, P_CS = 6 };

template <int P> struct Prim {
    static constexpr bool in = P != P_SEND && P != P_CS;  // reads the receive slot
    static constexpr bool local = P == P_SEND || P == P_RRS || P == P_RRCS || P == P_RRC || P == P_CS;
    static constexpr bool reduce = P == P_RRS || P == P_RRCS || P == P_RRC;
    static constexpr bool out = P != P_SEND && P != P_RRS;  // writes the output
    static constexpr bool send = P != P_RECV && P != P_RRC;  // writes the successor's slot
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

StagedKernel pick_staged_kernel(int dt, int op) {
    switch (dt) {
        case RR_INT32: return staged_kernel_for_op<DT_I32>(op);
        case RR_FP32: return staged_kernel_for_op<DT_F32>(op);
        case RR_BF16: return staged_kernel_for_op<DT_BF16>(op);
        case RR_FP16: return staged_kernel_for_op<DT_F16>(op);
        default: return nullptr;
    }
}

}  // namespace rr
