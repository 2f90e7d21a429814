// qmoe_decode_k4.hip -- the 4-bit instantiations of the decode and Q/K/V kernels.
#include "qmoe_decode_dev.h"

namespace qmoe {

DecodeKernel decode_kernel_b4(int variant) {
  switch (variant) {
    case 1: return decode_kernel<4, true, false>;
    case 2: return decode_kernel<4, true, true>;
    case 3: return decode_kernel<4, false, false, true>;
    default: return decode_kernel<4, false>;
  }
}

QkvKernel qkv_kernel_b4() { return qkv_kernel<4>; }
QkvKernel qkv_batched_kernel_b4() { return qkv_batched_kernel<4>; }

}  // namespace qmoe
