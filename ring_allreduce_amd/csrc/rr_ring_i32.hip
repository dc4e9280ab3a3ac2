// rr_ring_i32.hip -- the in-place ring kernels for int32 elements.
#include "rr_ring_kernel.hpp"

namespace rr {

RingKernel pick_ring_kernel_i32(int op, int block, bool alternate) {
    return ring_kernel_for_type<DT_I32>(op, block, alternate);
}

}  // namespace rr
