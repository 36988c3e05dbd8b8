// k_gemv_bf_gu.hip -- instantiations of the expert GEMV for bf16 experts, gate/up + SwiGLU.
#include "gemv_impl.h"

namespace moe {

hipError_t gemv_bf_gu(const GemvArgs& a, int ws_dtype, int ntmax, int act_bf16, unsigned blocks,
                      hipStream_t s) {
  const int k = a.geo.kc;
  const bool same = !a.has_shared || ws_dtype == MOE_BF16;
  const bool bf = a.has_shared && ws_dtype == MOE_BF16;
  if (!same && !bf) return hipErrorInvalidValue;
  if (k == 8) return gemv_go<MOE_BF16, 8, MOE_BF16, 8, false>(a, ntmax, act_bf16, blocks, s);
  if (k == 16) return gemv_go<MOE_BF16, 16, MOE_BF16, 16, false>(a, ntmax, act_bf16, blocks, s);
  if (k == 32) return gemv_go<MOE_BF16, 32, MOE_BF16, 32, false>(a, ntmax, act_bf16, blocks, s);
  if (k == 64) return gemv_go<MOE_BF16, 64, MOE_BF16, 64, false>(a, ntmax, act_bf16, blocks, s);
  if (k == 96) return gemv_go<MOE_BF16, 96, MOE_BF16, 96, false>(a, ntmax, act_bf16, blocks, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
