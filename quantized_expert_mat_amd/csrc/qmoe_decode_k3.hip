// qmoe_decode_k3.hip -- the 3-bit instantiations of the decode and Q/K/V kernels.
#include "qmoe_decode_dev.h"

namespace qmoe {

DecodeKernel decode_kernel_b3(int variant) {
  switch (variant) {
    case 1: return decode_kernel<3, true, false>;
    case 2: return decode_kernel<3, true, true>;
    case 3: return decode_kernel<3, false, false, true>;
    default: return decode_kernel<3, false>;
  }
}

QkvKernel qkv_kernel_b3() { return qkv_kernel<3>; }
QkvKernel qkv_batched_kernel_b3() { return qkv_batched_kernel<3>; }

}  // namespace qmoe
