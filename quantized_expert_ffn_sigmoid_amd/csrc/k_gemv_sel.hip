// k_gemv_sel.hip -- routed gate/up + SwiGLU of a one-token decode step, with
// the router's selection and the grouping run inside every block (gfx950).
//
// The selection ("colibri" README, "What's implemented": sigmoid noaux_tc
// router; "Glacial" page: softmax top-k) of one token is a few microseconds of
// one block's work on 256 logits, and its result -- which expert each routed
// block streams -- is needed by every block of the gate/up launch.  Rather
// than a launch of its own, every block computes it from the logits into LDS
// (the same deterministic code, so every block holds the same bits), reads its
// own slot record there, and block 0 also writes the routing and grouping out
// for the later launches and the caller.  No block reads another block's
// writes, so no cross-block synchronisation is needed.
#include "gemv_impl.h"

namespace moe {

namespace {

constexpr int kSelMaxSlots = kDecodeTokens * kMaxTopK;
constexpr int kMaxSelExperts = 4 * 64;   // experts per lane (EPL) at most 4

// The block's copy of the routing and grouping, in the ring area of the LDS
// (dead once the block knows its slot, before the ring fills).
struct __attribute__((aligned(16))) SelScratch {
  int32_t idx[kSelMaxSlots];
  float w[kSelMaxSlots];
  int32_t counts[kMaxExperts];
  int32_t offsets[kMaxExperts + 4];
  int32_t active[kMaxExperts];
  int32_t n_active[4];
  int32_t entries[kSelMaxSlots];
  int32_t inverse[kSelMaxSlots];
  int32_t pos_e[kSelMaxSlots];
  int32_t slot_tab[kSelMaxSlots * kSlotRec];
};
static_assert(sizeof(SelScratch) <= sizeof(RingLds::ring), "selection scratch fits the ring area");

template <int WR, int KR, int EPL, int ABF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_gemv_sel(
    GemvArgs a, PreArgs p) {
  __shared__ RingLds lds;
  SelScratch& S = *reinterpret_cast<SelScratch*>(&lds.ring[0][0][0]);
  const int T = p.T, F = T * p.sp.K, E = p.sp.E;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Wave 0 selects: its candidate loads go out first.  The token's
  // activation slice (sliced row 0: every routed row of a one-token step is
  // token 0) does not depend on the routing: its loads follow, so that they
  // have landed when the block's ring starts, and the ring's whole first fill
  // is issued at once.
  double ra[EPL], rb[EPL];
  if (wave == 0) {
    if (p.sp.softmax) select_load<EPL, true>(p.sp, p.zin, p.bias, nullptr, ra, rb);
    else select_load<EPL, false>(p.sp, p.zin, p.bias, p.sp.zsc, ra, rb);
  }
  constexpr int GPL = KR / Fmt<WR>::EPG;
  float xpre[KR], gpre[GPL];
  {
    const int64_t xo0 = 0;
    float (&xv)[1][KR] = *reinterpret_cast<float (*)[1][KR]>(&xpre[0]);
    slices_sliced_load<Fmt<WR>::EPG, KR, 1, ABF16>(a.x, &xo0, 1, xv);
  }
  SlotTables tb;
  tb.slot_tab = S.slot_tab;
  tb.n_tab = p.tb.n_tab;
  tb.pos_e = S.pos_e;
  if (wave == 0) {
    // the selection and the grouping of the token, in this wave alone
    if (p.sp.softmax) select_from<EPL, true>(p.sp, false, ra, rb, S.idx, S.w, nullptr);
    else select_from<EPL, false>(p.sp, p.sp.zsc != nullptr, ra, rb, S.idx, S.w, nullptr);
    bucket_one_token<(kMaxSelExperts + 63) / 64>(p.sp.K, E, S.idx, S.counts, S.offsets,
                                                 S.entries, S.inverse, S.active, S.n_active, tb);
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    // the routing and the grouping for the caller and the later launches
    for (int i = threadIdx.x; i < F; i += kThreads) {
      p.idx[i] = S.idx[i];
      p.w[i] = S.w[i];
      p.entries[i] = S.entries[i];
      p.inverse[i] = S.inverse[i];
      if (p.tb.pos_e) p.tb.pos_e[i] = S.pos_e[i];
    }
    for (int e = threadIdx.x; e < E; e += kThreads) {
      p.counts[e] = S.counts[e];
      p.offsets[e] = S.offsets[e];
      p.active[e] = S.active[e];
    }
    if (threadIdx.x == 0) {
      p.offsets[E] = S.offsets[E];
      p.n_active[0] = S.n_active[0];
    }
    if (p.tb.slot_tab)
      for (int i = threadIdx.x; i < tb.n_tab * kSlotRec; i += kThreads)
        p.tb.slot_tab[i] = S.slot_tab[i];
  }
  // the block's slot record, from its own copy
  GemvArgs b = a;
  b.src.slot_tab = S.slot_tab;
  b.src.pos_e = S.pos_e;
  b.src.active = S.active;
  b.src.n_active = S.n_active;
  b.src.offsets = S.offsets;
  b.src.entries = S.entries;
  BlockWork bw;
  const bool ok = block_work(b, bw, blockIdx.x);
  // every wave holds its record before the ring overwrites the scratch
  __syncthreads();
  if (!ok) return;
  {
    float (&xv)[1][KR] = *reinterpret_cast<float (*)[1][KR]>(&xpre[0]);
    float (&gv)[1][GPL] = *reinterpret_cast<float (*)[1][GPL]>(&gpre[0]);
    slice_finish<Fmt<WR>::EPG, KR, 1, ABF16>(xv, gv);
  }
  run_block<WR, KR, 1, ABF16, false, true>(b, bw, lds, xpre, gpre);
}

template <int WR, int KR, int EPL>
hipError_t go(const GemvArgs& a, const PreArgs& p, int act_bf16, unsigned blocks, hipStream_t s) {
  if (act_bf16)
    hipLaunchKernelGGL((k_gemv_sel<WR, KR, EPL, 1>), dim3(blocks), dim3(kThreads), 0, s, a, p);
  else
    hipLaunchKernelGGL((k_gemv_sel<WR, KR, EPL, 0>), dim3(blocks), dim3(kThreads), 0, s, a, p);
  return hipGetLastError();
}

}  // namespace

// The compiled (format, slice length, experts per lane) combinations: the
// GLM-scale decode layer (int4 or int8 experts, H 6144, 256 experts) and the
// Granite-shaped one (bf16 experts, H 1024, 32 experts).
bool gemv_sel_supported(const moe_layer_desc& d, int32_t T) {
  MatGeo g;
  if (T != 1 || !make_geo(d.expert_dtype, d.hidden, g) || g.lpr != 64) return false;
  const int epl = (d.n_experts + 63) / 64;
  if (d.expert_dtype == MOE_I4 || d.expert_dtype == MOE_I8) return g.kc == 96 && epl == 4;
  if (d.expert_dtype == MOE_BF16) return g.kc == 16 && epl == 1;
  return false;
}

hipError_t launch_gemv_sel(GemvArgs a, const PreArgs& p, int dtype, int act_bf16,
                           hipStream_t s) {
  int ntmax = 1, sd = dtype;
  a.has_shared = 0;
  const long long blocks = plan_gemv(a, false, dtype, sd, 1, false, ntmax);
  if (blocks <= 0 || a.per_token || a.geo.lpr != 64) return hipErrorInvalidValue;
  const unsigned nblk = (unsigned)blocks;
  if (dtype == MOE_I4 && a.geo.kc == 96) return go<MOE_I4, 96, 4>(a, p, act_bf16, nblk, s);
  if (dtype == MOE_I8 && a.geo.kc == 96) return go<MOE_I8, 96, 4>(a, p, act_bf16, nblk, s);
  if (dtype == MOE_BF16 && a.geo.kc == 16) return go<MOE_BF16, 16, 1>(a, p, act_bf16, nblk, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
