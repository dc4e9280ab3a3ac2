// rr_ring_f16.hip -- the in-place ring kernels for fp16 elements.
#include "rr_ring_kernel.hpp"

namespace rr {

RingKernel pick_ring_kernel_f16(int op, int block, bool alternate) {
    return ring_kernel_for_type<DT_F16>(op, block, alternate);
}

}  // namespace rr
