// down_fused.h -- down projections and the combine in one launch, for a decode
// step of one token (gfx950).
//
// The layer's output is out[o] = sum_j w_j * (down_j h_j)[o] + (down_s h_s)[o]
// ("colibri" README, "What's implemented": routed_scaling_factor-weighted
// combine of the routed experts plus the shared expert).  With one token the
// k routed rows of an output o and the shared expert's row are all the work
// behind out[o], so a block that owns a range of output rows computes them
// completely: no per-expert output rows go to memory and no separate combine
// launch runs.
//
// A block of kWaves waves owns rows [o0, o0 + R).  Wave w streams, through
// its LDS ring (the decode GEMV's ring), the down rows of the routed slots
// w and w + kWaves (up to two units) and granules [w GS, (w + 1) GS) of the
// shared expert's down rows, for every row of the block.  For each row a lane
// forms one value, sum_u c_u acc_u + acc_s (c_u = w_u * scale_u[o] with the
// code unit), and one 64-lane sum gives the wave's part of out[o]; the parts
// of the waves are added in wave order (deterministic) and written with the
// residual when a stack asks for it.
#pragma once

#include "gemv_impl.h"

namespace moe {

constexpr int kFusedMaxRows = 64;   // output rows per block
constexpr int kFusedMaxUnits = 2 * kWaves;

struct __attribute__((aligned(16))) FusedLds {
  uint8_t ring[kWaves][kRing][1024];
  float scale[kFusedMaxUnits][kFusedMaxRows];   // routed row scales, by unit
  float part[kWaves][kFusedMaxRows];            // per-wave part of each row
};

struct DownFusedArgs {
  ExpertSetDev w, ws;
  int32_t has_shared, H, I, Is, R;
  const int32_t* slot_tab;   // decode slot records (kSlotRec ints per slot)
  int32_t n_slots;           // records in slot_tab (<= kFusedMaxUnits)
  const float* topk_w;       // [k] routing weights of the token
  const void* h;             // routed h rows [slot][I], sliced for the down matrix
  const void* h_s;           // shared h [Is], sliced for the shared down matrix
  const float* s_pre;        // nullable: the shared expert's output [H], formed by the
                             // gate/up launch (then no shared granules stream here)
  const float* residual;     // nullable: out = residual + y
  float* out;                // [H]
  float* y_copy;             // nullable: y (the layer output without residual)
};

// Pieces of 16 bytes per lane that hold NG granules of a sliced activation
// row (fp32 or bf16 activations, EPG elements per granule).
template <int EPG, int NG, int ABF16>
constexpr int slice_pieces() {
  return NG * (EPG / (16 / (ABF16 ? 2 : 4)));
}

// Loads NG granules of the sliced activation row, starting at granule g0 of
// the lane's slice (lane j's granule g holds elements (g * 64 + j) * EPG ..),
// as raw pieces: the loads only, so that the caller can issue more loads
// before the first use of these.
template <int EPG, int NG, int ABF16>
__device__ __forceinline__ void slice_raw_load(const void* src, int g0,
                                               u32x4 (&raw)[slice_pieces<EPG, NG, ABF16>()]) {
  constexpr int PPC = slice_pieces<EPG, 1, ABF16>();
  const int j = threadIdx.x & 63;
  const uint8_t* row = reinterpret_cast<const uint8_t*>(src);
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int c = 0; c < PPC; ++c)
      raw[g * PPC + c] =
          *reinterpret_cast<const u32x4*>(row + ((int64_t)((g0 + g) * PPC + c) * 64 + j) * 16);
}

// The activations of the raw pieces as floats, and each granule's sum.
template <int EPG, int NG, int ABF16>
__device__ __forceinline__ void slice_raw_finish(const u32x4 (&raw)[slice_pieces<EPG, NG, ABF16>()],
                                                 float (&x)[NG * EPG], float (&gs)[NG]) {
  constexpr int PPC = slice_pieces<EPG, 1, ABF16>();
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < PPC; ++c) {
      const u32x4 v = raw[g * PPC + c];
      if constexpr (ABF16) {
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float lo = __uint_as_float(wv[d] << 16), hi = __uint_as_float(wv[d] & 0xFFFF0000u);
          x[g * EPG + c * 8 + 2 * d] = lo;
          x[g * EPG + c * 8 + 2 * d + 1] = hi;
          s += lo + hi;
        }
      } else {
        const float f[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                            __uint_as_float(v.w)};
#pragma unroll
        for (int d = 0; d < 4; ++d) x[g * EPG + c * 4 + d] = f[d];
        s += (f[0] + f[1]) + (f[2] + f[3]);
      }
    }
    gs[g] = s;
  }
}

// One wave's stream: NU routed units (slots u0, u0 + kWaves) and GS shared
// granules of every block row.  Items of row i, in order: the slots of unit
// 0's row (granule-major, int8 halves inner), unit 1's, then the shared
// granules; ring slot n holds item n.
template <int WR, int KR, int WS, int GS, int NU, int ABF16, int PR, int PS>
__device__ void fused_wave(const DownFusedArgs& a, int o0, int R, FusedLds& L, const int (&ue)[2],
                           const float (&uw)[2], const u32x4 (&hraw)[2][PR],
                           const u32x4 (&sraw)[PS]) {
  using FR = Fmt<WR>;
  using FS = Fmt<WS>;
  constexpr int GPL = KR / FR::EPG;
  constexpr int HPG = FR::GB >= 16 ? FR::GB / 16 : 1;
  constexpr int SR = GPL * HPG;          // ring slots per routed row
  constexpr int S = NU * SR + GS;        // slots per block row
  static_assert(FR::GB == 16 || WR == MOE_I8, "routed granules of 16 or 32 bytes");
  static_assert(GS == 0 || FS::GB == 16, "shared granules of 16 bytes");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (S == 0) {
    // nothing to stream: the wave's part of every row is zero
    if (lane < R) L.part[wave][lane] = 0.f;
    return;
  }
  const int64_t rb_r = (int64_t)(a.I / FR::EPG) * FR::GB;
  const int64_t rb_s = (int64_t)(a.Is / FS::EPG) * FS::GB;
  const uint8_t* wu[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    wu[u] = a.w.dn + (int64_t)(u < NU ? ue[u] : 0) * a.w.dn_stride + (int64_t)o0 * rb_r +
            lane * FR::GB;
  const uint8_t* wsb = a.has_shared ? a.ws.dn + (int64_t)o0 * rb_s + (int64_t)wave * GS * 64 * 16 + lane * 16
                                    : nullptr;
  uint8_t* ring = &L.ring[wave][0][0];
  const int total = R * S;
  auto slot_addr = [&](int n) -> const uint8_t* {
    const int i = n / S, idx = n - i * S;
    if (NU > 0 && idx < NU * SR) {
      const int u = idx / SR, gh = idx - u * SR;
      const int g = gh / HPG, hh = gh - g * HPG;
      const uint8_t* b = u == 0 ? wu[0] : wu[1];
      return b + (int64_t)i * rb_r + g * (64 * FR::GB) + hh * 16;
    }
    const int gsl = idx - NU * SR;
    return wsb + (int64_t)i * rb_s + gsl * (64 * 16);
  };
  auto issue = [&](int n) {
    const uint8_t* p = n < total ? slot_addr(n) : (NU > 0 ? wu[0] : wsb);
    __builtin_amdgcn_global_load_lds(p, (lds_ptr_t)(ring + (n & (kRing - 1)) * 1024), 16, 0, 2);
  };

  // activations: the units' h rows and the wave's granules of h_s, loaded
  // by the caller (they have landed); the ring's whole first fill goes out
  float xr[NU > 0 ? NU : 1][KR], gr[NU > 0 ? NU : 1][GPL];
  float xs[GS > 0 ? GS * FS::EPG : 1], gss[GS > 0 ? GS : 1];
  static_assert(PR == slice_pieces<FR::EPG, GPL, ABF16>(), "routed h pieces");
#pragma unroll
  for (int u = 0; u < NU; ++u) slice_raw_finish<FR::EPG, GPL, ABF16>(hraw[u], xr[u], gr[u]);
  if constexpr (GS > 0) {
    static_assert(PS == slice_pieces<FS::EPG, GS, ABF16>(), "shared h pieces");
    float (&xsv)[GS * FS::EPG] = *reinterpret_cast<float (*)[GS * FS::EPG]>(&xs[0]);
    float (&gsv)[GS] = *reinterpret_cast<float (*)[GS]>(&gss[0]);
    slice_raw_finish<FS::EPG, GS, ABF16>(sraw, xsv, gsv);
  }
#pragma unroll
  for (int n = 0; n < kRing; ++n) issue(n);

  auto read_slot = [&](int n) {
    return *reinterpret_cast<const u32x4*>(ring + (n & (kRing - 1)) * 1024 + lane * 16);
  };
  u32x4 vnext = {0u, 0u, 0u, 0u};
  if (total > 0) {
    if (total - 1 >= kRing - 2) wait_vmcnt<kRing - 2>();
    else wait_vmcnt<0>();
    vnext = read_slot(0);
  }
  for (int i = 0; i < R; ++i) {
    float acc[NU > 0 ? NU : 1], accs = 0.f;
#pragma unroll
    for (int u = 0; u < (NU > 0 ? NU : 1); ++u) acc[u] = 0.f;
#pragma unroll
    for (int idx = 0; idx < S; ++idx) {
      const int t = i * S + idx;
      const u32x4 v = vnext;
      if (t + 1 < total) {
        if (total - t - 2 >= kRing - 2) wait_vmcnt<kRing - 2>();
        else wait_vmcnt<0>();
        vnext = read_slot(t + 1);
      }
      const uint32_t g4[4] = {v.x, v.y, v.z, v.w};
      if (idx < NU * SR) {
        const int u = idx / SR, gh = idx % SR;
        const int g = gh / HPG, hh = gh % HPG;
        float a1[1] = {acc[u]};
        const float (&xu)[1][KR] = *reinterpret_cast<const float (*)[1][KR]>(&xr[u][0]);
        if constexpr (HPG == 1) granule_fma<WR, 1, KR>(g4, xu, g, a1);
        else i8_half_fma<1, KR>(g4, xu, g * FR::EPG + 16 * hh, a1);
        if constexpr (WR != MOE_BF16) {
          if (hh == HPG - 1) a1[0] = fmaf(-FR::OFF * FR::UNIT, gr[u][g], a1[0]);
        }
        acc[u] = a1[0];
      } else if constexpr (GS > 0) {
        const int g = idx - NU * SR;
        float a1[1] = {accs};
        const float (&xsv)[1][GS * FS::EPG] = *reinterpret_cast<const float (*)[1][GS * FS::EPG]>(&xs[0]);
        granule_fma<WS, 1, GS * FS::EPG>(g4, xsv, g, a1);
        if constexpr (WS != MOE_BF16) a1[0] = fmaf(-FS::OFF * FS::UNIT, gss[g], a1[0]);
        accs = a1[0];
      }
      // the slot's data has fed the FMAs: refill it
      asm volatile("" : "+v"(accs) : "v"(v.x), "v"(v.w) : "memory");
#pragma unroll
      for (int u = 0; u < (NU > 0 ? NU : 1); ++u) asm volatile("" : "+v"(acc[u]) : : "memory");
      if (t + kRing < total) issue(t + kRing);
    }
    float val = accs;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float c = uw[u];
      if constexpr (WR != MOE_BF16) c *= L.scale[wave + u * kWaves][i] * (1.0f / FR::UNIT);
      val = fmaf(c, acc[u], val);
    }
    val = group_sum(val, 64);
    if (lane == 0) L.part[wave][i] = val;
  }
  if (total < kRing) wait_vmcnt<0>();
}

// The kernel: every block stages its units' row scales, each wave streams
// its units (two, one or none routed; the shared granules), then the block
// adds the parts of its waves.
template <int WR, int KR, int WS, int GS, int ABF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_down_fused(
    DownFusedArgs a) {
  __shared__ FusedLds L;
  const int o0 = blockIdx.x * a.R;
  const int R = min(a.R, a.H - o0);
  if (R <= 0) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the wave's units: slots wave and wave + kWaves that hold an expert
  // (the grouping fills slots 0 .. n_active - 1, so the valid slots of a wave
  // form a prefix of its two)
  int ue[2] = {0, 0}, uh[2] = {0, 0};
  float uw[2] = {0.f, 0.f};
  int nu = 0;
  // The h rows go out first: a one-token step's grouping gives every active
  // expert one row, in expert order, so slot s's row is bucket position s
  // (checked against the records below).  Clamped to a row that exists.
  using FR = Fmt<WR>;
  constexpr int GPL = KR / FR::EPG;
  constexpr int PR = slice_pieces<FR::EPG, GPL, ABF16>();
  constexpr int PS = GS > 0 ? slice_pieces<Fmt<WS>::EPG, GS, ABF16>() : 1;
  constexpr int ABR = ABF16 ? 2 : 4;
  const int last = max(a.n_slots, 1) - 1;
  u32x4 hraw[2][PR], sraw[PS];
  auto load_h = [&](int u, int pos) {
    slice_raw_load<FR::EPG, GPL, ABF16>(
        reinterpret_cast<const uint8_t*>(a.h) + (int64_t)pos * a.I * ABR, 0, hraw[u]);
  };
#pragma unroll
  for (int u = 0; u < 2; ++u) load_h(u, min(wave + u * kWaves, last));
  if constexpr (GS > 0) slice_raw_load<Fmt<WS>::EPG, GS, ABF16>(a.h_s, wave * GS, sraw);
  if (a.n_slots > 0) {
    // one round trip: lanes 0 and 1 read the two records (indexes clamped
    // to a record that exists), every lane a routing weight of the token (a
    // one-token step's record names its weight by its flat slot, < n_slots);
    // a record past the active experts holds only its expert field, -1
    const int su = min(wave + (lane & 1) * kWaves, a.n_slots - 1);
    const int4 rv = *reinterpret_cast<const int4*>(a.slot_tab + (int64_t)su * kSlotRec);
    const float wl = a.topk_w[min(lane, a.n_slots - 1)];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int rx = __builtin_amdgcn_readlane(rv.x, u);
      const int ry = __builtin_amdgcn_readlane(rv.y, u);
      const int rw = min(max(__builtin_amdgcn_readlane(rv.w, u), 0), a.n_slots - 1);
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), rw));
      if (wave + u * kWaves < a.n_slots && rx >= 0 && nu == u) {
        ue[u] = rx;
        uh[u] = ry;
        uw[u] = w;
        nu = u + 1;
      }
    }
  }
  // h was requested before the records and has landed with them; said
  // here for every path, so that the compiler's own wait before h's first
  // use does not become a wait for the ring's whole first fill
  wait_vmcnt<0>();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    ue[u] = __builtin_amdgcn_readfirstlane(ue[u]);
    uh[u] = __builtin_amdgcn_readfirstlane(uh[u]);
    uw[u] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(uw[u])));
  }
  nu = __builtin_amdgcn_readfirstlane(nu);
  // a record whose row is not at its slot's position (not a one-token
  // grouping): that row again, from where the record puts it, waited for
  // here (no h load is pending past this point)
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (u < nu && uh[u] != wave + u * kWaves) {
      load_h(u, uh[u]);
      wait_vmcnt<0>();
    }
  // row scales of the wave's units, by direct loads into LDS (lane l fills
  // entry l; lanes past the block's rows reload its last row); the ring's
  // first wait covers them, as they are issued before its loads
  if constexpr (WR != MOE_BF16) {
    for (int u = 0; u < nu; ++u) {
      const float* S = reinterpret_cast<const float*>(a.w.dns + (int64_t)ue[u] * a.w.dns_stride);
      __builtin_amdgcn_global_load_lds(S + o0 + min(lane, R - 1),
                                       (lds_ptr_t)&L.scale[wave + u * kWaves][0], 4, 0, 0);
    }
  }
  if (nu == 2) fused_wave<WR, KR, WS, GS, 2, ABF16, PR, PS>(a, o0, R, L, ue, uw, hraw, sraw);
  else if (nu == 1) fused_wave<WR, KR, WS, GS, 1, ABF16, PR, PS>(a, o0, R, L, ue, uw, hraw, sraw);
  else fused_wave<WR, KR, WS, GS, 0, ABF16, PR, PS>(a, o0, R, L, ue, uw, hraw, sraw);
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += kThreads) {
    float y = L.part[0][r];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) y += L.part[w][r];
    const int o = o0 + r;
    if (a.s_pre) y += a.s_pre[o];
    if (a.y_copy) a.y_copy[o] = y;
    a.out[o] = a.residual ? a.residual[o] + y : y;
  }
}

}  // namespace moe
