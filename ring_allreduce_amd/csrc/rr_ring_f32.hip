// rr_ring_f32.hip -- the in-place ring kernels for fp32 elements.
#include "rr_ring_kernel.hpp"

namespace rr {

RingKernel pick_ring_kernel_f32(int op, int block, bool alternate) {
    return ring_kernel_for_type<DT_F32>(op, block, alternate);
}

}  // namespace rr
