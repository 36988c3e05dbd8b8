// k_gemv_i8_dn.hip -- instantiations of the expert GEMV for int8 experts, down projection.
#include "gemv_impl.h"

namespace moe {

hipError_t gemv_i8_dn(const GemvArgs& a, int ws_dtype, int ntmax, int act_bf16, unsigned blocks,
                      hipStream_t s) {
  const int k = a.geo.kc;
  const bool same = !a.has_shared || ws_dtype == MOE_I8;
  const bool bf = a.has_shared && ws_dtype == MOE_BF16;
  if (!same && !bf) return hipErrorInvalidValue;
  if (k == 32 && same) return gemv_go<MOE_I8, 32, MOE_I8, 32, true>(a, ntmax, act_bf16, blocks, s);
  if (k == 32 && bf) return gemv_go<MOE_I8, 32, MOE_BF16, 32, true>(a, ntmax, act_bf16, blocks, s);
  if (k == 64 && same) return gemv_go<MOE_I8, 64, MOE_I8, 64, true>(a, ntmax, act_bf16, blocks, s);
  if (k == 64 && bf) return gemv_go<MOE_I8, 64, MOE_BF16, 64, true>(a, ntmax, act_bf16, blocks, s);
  if (k == 96 && same) return gemv_go<MOE_I8, 96, MOE_I8, 96, true>(a, ntmax, act_bf16, blocks, s);
  if (k == 96 && bf) return gemv_go<MOE_I8, 96, MOE_BF16, 96, true>(a, ntmax, act_bf16, blocks, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
