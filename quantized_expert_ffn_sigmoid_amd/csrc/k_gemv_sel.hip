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
//
// While one wave selects, the block's other waves would idle for several
// microseconds before any weight of the routed experts can be requested.
// With a bf16 shared expert they spend that time on the shared expert's down
// projection (its h is complete: the logits launch formed it), each block
// over its share of the output rows, and the down launch adds that output
// instead of streaming the shared weights itself.  Their loads go out after
// the selecting wave's candidate loads (a barrier between the two), so that
// the selection's inputs are not queued behind them.
#include "down_fused.h"

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

// The shared expert's down rows [o0, o1) of this block (o0 = block * rpb),
// out[o] = sum_c down_s[o][c] h_s[c], by waves 1 .. kWaves - 1: wave w takes
// rows o0 + w - 1, o0 + w - 1 + (kWaves - 1), ...  A lane holds granules j,
// j + 64, j + 128, j + 192 of a kSdnIs-wide row (8 bf16 weights each) and the
// matching 32 values of h; the rows of a pass are requested together, then
// each is dotted, summed over the wave and written.  load_x issues the wave's
// other loads behind the first pass's rows (loads complete in issue order, so
// the rows are not held up behind them).
template <int ABF16, class XL>
__device__ __forceinline__ void shared_down_rows(const PreArgs& p, int wave, XL&& load_x) {
  constexpr int EPG = Fmt<MOE_BF16>::EPG;
  constexpr int GPL = kSdnIs / kWave / EPG;
  constexpr int KSL = GPL * EPG;
  constexpr int RW = 4;              // rows per pass
  constexpr int NW = kWaves - 1;     // waves that take rows
  constexpr int64_t RB = (int64_t)kSdnIs * 2;
  static_assert(GPL * EPG * kWave == kSdnIs, "whole granules per lane");
  const int lane = threadIdx.x & 63;
  const int o0 = (int)blockIdx.x * p.sdn_rpb;
  const int o1 = min(p.H, o0 + p.sdn_rpb);
  if (o0 + wave - 1 >= o1) {
    load_x();
    return;
  }
  const uint8_t* wl = p.sdn + lane * 16;
  u32x4 hr[slice_pieces<EPG, GPL, ABF16>()];
  slice_raw_load<EPG, GPL, ABF16>(p.sdn_h, 0, hr);
  auto pass = [&](int r0, auto first) {
    u32x4 v[RW][GPL];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int o = r0 + i * NW;   // wave-uniform
#pragma unroll
      for (int g = 0; g < GPL; ++g)
        v[i][g] = o < o1 ? __builtin_nontemporal_load(
                               reinterpret_cast<const u32x4*>(wl + (int64_t)o * RB + g * 1024))
                         : u32x4{0u, 0u, 0u, 0u};
    }
    if constexpr (decltype(first)::value) load_x();
    float x[1][KSL], gs[GPL];
    slice_raw_finish<EPG, GPL, ABF16>(hr, x[0], gs);
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int o = r0 + i * NW;
      float acc[1] = {0.f};
#pragma unroll
      for (int g = 0; g < GPL; ++g) {
        const uint32_t gr[4] = {v[i][g].x, v[i][g].y, v[i][g].z, v[i][g].w};
        granule_fma<MOE_BF16, 1, KSL>(gr, x, g, acc);
      }
      const float sum = group_sum(acc[0], 64);
      if (o < o1 && lane == 0) p.sdn_out[o] = sum;
    }
  };
  pass(o0 + wave - 1, std::true_type{});
  for (int r0 = o0 + wave - 1 + NW * RW; r0 < o1; r0 += NW * RW) pass(r0, std::false_type{});
}

template <int WR, int KR, int EPL, int ABF16, bool SDN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_gemv_sel(
    GemvArgs a, PreArgs p) {
  __shared__ RingLds lds;
  SelScratch& S = *reinterpret_cast<SelScratch*>(&lds.ring[0][0][0]);
  const int T = p.T, F = T * p.sp.K, E = p.sp.E;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Wave 0 selects: its candidate loads go out first.  The token's
  // activation slice (sliced row 0: every routed row of a one-token step is
  // token 0) does not depend on the routing: its loads follow (in the other
  // waves, behind their first shared down rows), so that they have landed
  // when the block's ring starts, and the ring's whole first fill is issued
  // at once.
  double ra[EPL], rb[EPL];
  if (wave == 0) {
    if (p.sp.softmax) select_load<EPL, true>(p.sp, p.zin, p.bias, nullptr, ra, rb);
    else select_load<EPL, false>(p.sp, p.zin, p.bias, p.sp.zsc, ra, rb);
  }
  constexpr int GPL = KR / Fmt<WR>::EPG;
  float xpre[KR], gpre[GPL];
  auto load_x = [&]() {
    const int64_t xo0 = 0;
    float (&xv)[1][KR] = *reinterpret_cast<float (*)[1][KR]>(&xpre[0]);
    slices_sliced_load<Fmt<WR>::EPG, KR, 1, ABF16>(a.x, &xo0, 1, xv);
  };
  if constexpr (SDN) {
    if (wave == 0) load_x();
    // wave 0's candidate loads are out before the other waves' shared rows
    asm volatile("s_barrier" ::: "memory");
    if (wave > 0) shared_down_rows<ABF16>(p, wave, load_x);
  } else {
    load_x();
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

template <int WR, int KR, int EPL, bool SDN>
hipError_t go2(const GemvArgs& a, const PreArgs& p, int act_bf16, unsigned blocks, hipStream_t s) {
  if (act_bf16)
    hipLaunchKernelGGL((k_gemv_sel<WR, KR, EPL, 1, SDN>), dim3(blocks), dim3(kThreads), 0, s, a, p);
  else
    hipLaunchKernelGGL((k_gemv_sel<WR, KR, EPL, 0, SDN>), dim3(blocks), dim3(kThreads), 0, s, a, p);
  return hipGetLastError();
}

template <int WR, int KR, int EPL>
hipError_t go(const GemvArgs& a, PreArgs p, int act_bf16, unsigned blocks, hipStream_t s) {
  if (!p.sdn) return go2<WR, KR, EPL, false>(a, p, act_bf16, blocks, s);
  if (p.T != 1 || p.H <= 0 || !p.sdn_h || !p.sdn_out) return hipErrorInvalidValue;
  p.sdn_rpb = (int)((p.H + blocks - 1) / blocks);
  return go2<WR, KR, EPL, true>(a, p, act_bf16, blocks, s);
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
