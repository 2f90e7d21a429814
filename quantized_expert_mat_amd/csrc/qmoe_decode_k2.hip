// qmoe_decode_k2.hip -- the 2-bit instantiations of the decode and Q/K/V kernels.
#include "qmoe_decode_dev.h"

namespace qmoe {

DecodeKernel decode_kernel_b2(int variant) {
  switch (variant) {
    case 1: return decode_kernel<2, true, false>;
    case 2: return decode_kernel<2, true, true>;
    case 3: return decode_kernel<2, false, false, true>;
    default: return decode_kernel<2, false>;
  }
}

QkvKernel qkv_kernel_b2() { return qkv_kernel<2>; }
QkvKernel qkv_batched_kernel_b2() { return qkv_batched_kernel<2>; }

}  // namespace qmoe
