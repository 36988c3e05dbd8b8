// k_gemv_pre_gu.hip -- instantiations of the shared expert's gate/up + SwiGLU with
// leading blocks that run the router logits (decode).
#include "gemv_impl.h"

namespace moe {

hipError_t gemv_pre_gu(const GemvArgs& a, const PreArgs& p, int ws_dtype, int act_bf16,
                      unsigned blocks, hipStream_t s) {
  const int k = a.geo_s.kc;
  if (ws_dtype == MOE_BF16) {
    if (k == 8) return gemv_pre_go<MOE_BF16, 8, false>(a, p, act_bf16, blocks, s);
    if (k == 16) return gemv_pre_go<MOE_BF16, 16, false>(a, p, act_bf16, blocks, s);
    if (k == 32) return gemv_pre_go<MOE_BF16, 32, false>(a, p, act_bf16, blocks, s);
    if (k == 64) return gemv_pre_go<MOE_BF16, 64, false>(a, p, act_bf16, blocks, s);
    if (k == 96) return gemv_pre_go<MOE_BF16, 96, false>(a, p, act_bf16, blocks, s);
    if (k == 128) return gemv_pre_go<MOE_BF16, 128, false>(a, p, act_bf16, blocks, s);
    if (k == 112) return gemv_pre_go<MOE_BF16, 112, false>(a, p, act_bf16, blocks, s);
  } else if (ws_dtype == MOE_I4) {
    if (k == 32) return gemv_pre_go<MOE_I4, 32, false>(a, p, act_bf16, blocks, s);
    if (k == 64) return gemv_pre_go<MOE_I4, 64, false>(a, p, act_bf16, blocks, s);
    if (k == 96) return gemv_pre_go<MOE_I4, 96, false>(a, p, act_bf16, blocks, s);
    if (k == 128) return gemv_pre_go<MOE_I4, 128, false>(a, p, act_bf16, blocks, s);
  } else if (ws_dtype == MOE_I8) {
    if (k == 32) return gemv_pre_go<MOE_I8, 32, false>(a, p, act_bf16, blocks, s);
    if (k == 64) return gemv_pre_go<MOE_I8, 64, false>(a, p, act_bf16, blocks, s);
    if (k == 96) return gemv_pre_go<MOE_I8, 96, false>(a, p, act_bf16, blocks, s);
    if (k == 128) return gemv_pre_go<MOE_I8, 128, false>(a, p, act_bf16, blocks, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
