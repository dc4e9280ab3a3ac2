// rr_ring_bf16.hip -- the in-place ring kernels for bf16 elements.
#include "rr_ring_kernel.hpp"

namespace rr {

RingKernel pick_ring_kernel_bf16(int op, int block, bool alternate) {
    return ring_kernel_for_type<DT_BF16>(op, block, alternate);
}

}  // namespace rr
