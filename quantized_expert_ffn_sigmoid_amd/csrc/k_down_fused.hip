// k_down_fused.hip -- instantiations and launch of the one-token down
// projection + combine (down_fused.h).
#include "down_fused.h"

namespace moe {

namespace {

// Routed h slices per unit (KR elements per lane) and shared granules per
// wave (GS) that are compiled, by format.
bool fused_geometry(const moe_layer_desc& d, int& kr, int& gs) {
  const int wr = d.expert_dtype;
  if (wr != MOE_I4 && wr != MOE_I8 && wr != MOE_BF16) return false;
  if (!gemv_ring(wr, d.inter)) return false;
  kr = d.inter / kWave;
  const bool kr_ok = wr == MOE_BF16 ? (kr == 8 || kr == 32) : kr == 32;
  if (!kr_ok) return false;
  gs = 0;
  if (d.n_shared > 0) {
    const int Is = d.inter * d.n_shared;
    if (d.shared_dtype != MOE_BF16 || !gemv_ring(MOE_BF16, Is)) return false;
    const int gpl = Is / kWave / Fmt<MOE_BF16>::EPG;   // shared granules per lane
    if (gpl % kWaves) return false;
    gs = gpl / kWaves;
    if (gs != 1) return false;
  }
  return true;
}

template <int WR, int KR, int GS>
hipError_t go(const DownFusedArgs& a, int act_bf16, unsigned blocks, hipStream_t s) {
  if (act_bf16)
    hipLaunchKernelGGL((k_down_fused<WR, KR, MOE_BF16, GS, 1>), dim3(blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_down_fused<WR, KR, MOE_BF16, GS, 0>), dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool down_fused_supported(const moe_layer_desc& d, int32_t T) {
  int kr, gs;
  return T == 1 && d.top_k <= kFusedMaxUnits && fused_geometry(d, kr, gs);
}

hipError_t launch_down_fused(const moe_layer_desc& d, DownFusedArgs a, int act_bf16,
                             hipStream_t s) {
  int kr, gs;
  if (!fused_geometry(d, kr, gs) || a.n_slots > kFusedMaxUnits) return hipErrorInvalidValue;
  // the shared expert's output formed by the gate/up launch: only the routed
  // rows stream here
  if (a.s_pre) gs = 0;
  // rows per block: two blocks per CU over the output rows
  int R = (a.H + 511) / 512;
  if (R > kFusedMaxRows) R = kFusedMaxRows;
  a.R = R;
  const unsigned blocks = (unsigned)((a.H + R - 1) / R);
  const int wr = d.expert_dtype;
  if (wr == MOE_I4 && kr == 32) return gs ? go<MOE_I4, 32, 1>(a, act_bf16, blocks, s)
                                          : go<MOE_I4, 32, 0>(a, act_bf16, blocks, s);
  if (wr == MOE_I8 && kr == 32) return gs ? go<MOE_I8, 32, 1>(a, act_bf16, blocks, s)
                                          : go<MOE_I8, 32, 0>(a, act_bf16, blocks, s);
  if (wr == MOE_BF16 && kr == 8) return gs ? go<MOE_BF16, 8, 1>(a, act_bf16, blocks, s)
                                           : go<MOE_BF16, 8, 0>(a, act_bf16, blocks, s);
  if (wr == MOE_BF16 && kr == 32) return gs ? go<MOE_BF16, 32, 1>(a, act_bf16, blocks, s)
                                            : go<MOE_BF16, 32, 0>(a, act_bf16, blocks, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
