// qmoe_prefill.hip -- batched prefill through one MoE layer (expert-grouped bf16 GEMM).
#include <string>

#include "qmoe_internal.h"

namespace qmoe {

size_t prefill_ws_bytes(const moe_config& c, int T) {
  (void)c;
  (void)T;
  return 0;
}

moe_status prefill_forward(const moe_config& c, const moe_layer_weights* lw, int T,
                           const float* x, float* y, const float* sel_bias, const int32_t* boosted,
                           int32_t* idx_out, float* w_out, uint8_t* ws, size_t ws_bytes,
                           hipStream_t stream, std::string* msg) {
  (void)c; (void)lw; (void)T; (void)x; (void)y; (void)sel_bias; (void)boosted; (void)idx_out;
  (void)w_out; (void)ws; (void)ws_bytes; (void)stream;
  *msg = "MOE_F_PREFILL_BF16 is not built yet";
  return MOE_ERR_UNSUPPORTED;
}

}  // namespace qmoe
