// route_device.h -- device-side building blocks of the router selection and
// of the batch-union grouping, shared by the routing kernels (gfx950).
//
// Selection ("colibri" README, "What's implemented": DeepSeek-V3-style sigmoid
// router, noaux_tc, routed_scaling_factor): s = sigmoid(z), c = s + bias;
// n_group contiguous groups scored by the sum of their two largest c; the
// topk_group best groups kept; the top_k largest c among their experts chosen;
// weights s / sum(s) * scaling.  Softmax top-k (Granite layer, "Glacial" page):
// top_k largest z, weights softmax over them.  Every comparison prefers the
// larger value and, on equal values, the lower index.
#pragma once

#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ bool beats(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// ------------------------------------------------------- cross-lane moves
// DPP lane moves (register to register, no LDS round trip).  All patterns
// used here give every lane a valid source.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane j <-> 7-j within 8 lanes
constexpr int kDppMirror = 0x140;     // lane j <-> 15-j within 16 lanes

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = dpp_i<CTRL>((int)(b & 0xFFFFFFFFll));
  const int hi = dpp_i<CTRL>((int)(b >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// fp64 maximum and minimum as single instructions (the library fmax/fmin
// also canonicalize their operands; the values here are never NaN).
__device__ __forceinline__ double dmax(double a, double b) {
  double r;
  asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ double dmin(double a, double b) {
  double r;
  asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ double readlane_d(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFFll), lane);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// One all-reduce step of (value, index) best-of with the partner of a move
// (selects, no branches).
template <int CTRL>
__device__ __forceinline__ void argbest_step_dpp(double& v, int& i) {
  const double ov = dpp_d<CTRL>(v);
  const int oi = dpp_i<CTRL>(i);
  const bool take = beats(ov, oi, v, i);
  v = take ? ov : v;
  i = take ? oi : i;
}

// Wave-wide best (value, index), returned wave-uniform: every row of 16
// lanes reduces with register moves, then the four row results are compared
// through lane reads.
__device__ __forceinline__ void wave_argbest(double& v, int& i) {
  argbest_step_dpp<kDppXor1>(v, i);
  argbest_step_dpp<kDppXor2>(v, i);
  argbest_step_dpp<kDppHalfMirror>(v, i);
  argbest_step_dpp<kDppMirror>(v, i);
  double bv = readlane_d(v, 0);
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const double ov = readlane_d(v, 16 * r);
    const int oi = __builtin_amdgcn_readlane(i, 16 * r);
    const bool take = beats(ov, oi, bv, bi);
    bv = take ? ov : bv;
    bi = take ? oi : bi;
  }
  v = bv;
  i = bi;
}

// Wave-wide maximum of doubles, returned in every lane: DPP moves within rows
// of 16 lanes, then swaps of rows and of halves between two copies.
__device__ __forceinline__ double swap_max(double v, bool halves) {
  const long long b = __double_as_longlong(v);
  const uint32_t lo = (uint32_t)(b & 0xFFFFFFFFll), hi = (uint32_t)(b >> 32);
  uint32_t lo2, hi2, lo3, hi3;
  if (halves) {
    const auto pl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto ph = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    lo2 = pl[0]; lo3 = pl[1]; hi2 = ph[0]; hi3 = ph[1];
  } else {
    const auto pl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto ph = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    lo2 = pl[0]; lo3 = pl[1]; hi2 = ph[0]; hi3 = ph[1];
  }
  const double a = __longlong_as_double(((long long)hi2 << 32) | lo2);
  const double c = __longlong_as_double(((long long)hi3 << 32) | lo3);
  return dmax(a, c);
}
__device__ __forceinline__ double wave_max_d(double v) {
  v = dmax(v, dpp_d<kDppXor1>(v));
  v = dmax(v, dpp_d<kDppXor2>(v));
  v = dmax(v, dpp_d<kDppHalfMirror>(v));
  v = dmax(v, dpp_d<kDppMirror>(v));
  v = swap_max(v, false);
  return swap_max(v, true);
}

// Order-preserving 64-bit keys of doubles: key(a) > key(b) exactly when
// a > b (finite values; -0 below +0, which the selection never compares).
__device__ __forceinline__ uint64_t order_key(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ __forceinline__ double key_value(uint64_t k) {
  const uint64_t b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)b);
}

// Wave-wide maximum of 32-bit unsigned values, in every lane.  The lane
// moves give every lane a valid source, so the move's old value (0, the
// identity of the maximum) is never used; written this way the compiler
// folds each move into the maximum that consumes it.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<kDppXor1>(v));
  v = max(v, dpp_u<kDppXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  v = max(v, dpp_u<kDppMirror>(v));
  const auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(p16[0], p16[1]);
  const auto p32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(p32[0], p32[1]);
}

// The lanes holding the wave-wide maximum of 64-bit keys (a lane mask): the
// high words first; only when several lanes share the largest high word
// (the scores then agree to about 2^-20 of their value, rare) the low words
// of those lanes decide.
__device__ __forceinline__ uint64_t wave_max_key_lanes(uint64_t k) {
  const uint32_t hi = (uint32_t)(k >> 32);
  const uint32_t mh = wave_max_u32(hi);
  const uint64_t b = __ballot(hi == mh);
  if (__popcll(b) == 1) return b;
  const uint32_t ml = wave_max_u32(hi == mh ? (uint32_t)k : 0u);
  return __ballot(hi == mh && (uint32_t)k == ml);
}

// Two largest values (a >= b) merged with a partner's pair.
__device__ __forceinline__ void top2_merge(double& a, double& b, double oa, double ob) {
  const double hi = dmax(a, oa), lo = dmin(a, oa);
  b = dmax(lo, dmax(b, ob));
  a = hi;
}

template <int CTRL>
__device__ __forceinline__ void top2_step_dpp(double& a, double& b) {
  top2_merge(a, b, dpp_d<CTRL>(a), dpp_d<CTRL>(b));
}

// Top-2 all-reduce within aligned segments of lpg lanes (lpg a power of 2).
__device__ __forceinline__ void segment_top2(double& a, double& b, int lpg) {
  if (lpg >= 2) top2_step_dpp<kDppXor1>(a, b);
  if (lpg >= 4) top2_step_dpp<kDppXor2>(a, b);
  if (lpg >= 8) top2_step_dpp<kDppHalfMirror>(a, b);
  if (lpg >= 16) top2_step_dpp<kDppMirror>(a, b);
  if (lpg >= 32) top2_merge(a, b, __shfl_xor(a, 16, kWave), __shfl_xor(b, 16, kWave));
  if (lpg >= 64) top2_merge(a, b, __shfl_xor(a, 32, kWave), __shfl_xor(b, 32, kWave));
}

// Wave-wide two largest values (a >= b); lanes hold their local (a, b).
__device__ __forceinline__ void wave_top2(double& a, double& b) { segment_top2(a, b, 64); }

// The loads behind one token's selection candidates, issued but not used:
// lane l reads experts l*EPL .. l*EPL+EPL-1 (clamped to the last expert):
// the logits (softmax), the scores and biased scores the logits launch
// formed (sct), or the logits and the bias.  A caller can issue other loads
// before select_from consumes these.
template <int EPL, bool SOFTMAX>
__device__ __forceinline__ void select_load(const SelectParams& p, const double* __restrict__ zt,
                                            const float* __restrict__ bias, const double* sct,
                                            double (&ra)[EPL], double (&rb)[EPL]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int ec = min(lane * EPL + i, p.E - 1);
    if constexpr (SOFTMAX) {
      ra[i] = zt[ec];
      rb[i] = 0.0;
    } else if (sct) {
      ra[i] = sct[2 * ec];
      rb[i] = sct[2 * ec + 1];
    } else {
      ra[i] = zt[ec];
      rb[i] = bias ? (double)bias[ec] : 0.0;
    }
  }
}

// Selection for one token by one wave from the loads of select_load (sct:
// whether they were scores); writes its k expert indices and weights (rank
// order) to idx_out / w_out, and the indices also to idx_lds when given.
// Lane l holds experts l*EPL .. l*EPL+EPL-1, so a group is a run of
// consecutive lanes when EPL divides the group size.  Closed (or absent)
// experts carry -inf; the candidate loops use selects, and the loops over
// groups and ranks are wave-uniform.
template <int EPL, bool SOFTMAX>
__device__ __forceinline__ void select_from(const SelectParams& p, bool sct,
                                            const double (&ra)[EPL], const double (&rb)[EPL],
                                            int32_t* idx_out, float* w_out, int32_t* idx_lds) {
  const int lane = threadIdx.x & 63;
  const double NEG = -INFINITY;
  double c[EPL], sv[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const bool ok = lane * EPL + i < p.E;
    if constexpr (SOFTMAX) {
      sv[i] = ra[i];
      c[i] = ok ? ra[i] : NEG;
    } else if (sct) {
      // the token's scores, formed by the logits launch
      sv[i] = ra[i];
      c[i] = ok ? rb[i] : NEG;
    } else {
      const double s = 1.0 / (1.0 + exp(-ra[i]));
      sv[i] = s;
      c[i] = ok ? s + rb[i] : NEG;
    }
  }

  if (!SOFTMAX && p.topk_group < p.G) {
    const int per = p.E / p.G;
    const int lpg = per / EPL;
    const bool seg = per % EPL == 0 && lpg >= 1 && lpg <= kWave && (lpg & (lpg - 1)) == 0;
    if (seg) {
      // every lane's experts lie in one group: segmented top-2, then rank the
      // groups against each other through lane reads
      double a = NEG, b = NEG;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const double hi = dmax(a, c[i]), lo = dmin(a, c[i]);
        b = dmax(b, lo);
        a = hi;
      }
      segment_top2(a, b, lpg);
      const double gs = per == 1 ? a : a + b;
      const int my_g = (lane * EPL) / per;
      int rank = 0;
      for (int g = 0; g < p.G; ++g) {
        const double sg = readlane_d(gs, g * lpg);
        rank += beats(sg, g, gs, my_g) ? 1 : 0;
      }
      if (rank >= p.topk_group) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) c[i] = NEG;
      }
    } else {
      // general shapes: one group at a time
      double my_gs = NEG;
      for (int g = 0; g < p.G; ++g) {
        double a = NEG, b = NEG;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          const int e = lane * EPL + i;
          const double x = e / per == g ? c[i] : NEG;
          const double hi = dmax(a, x), lo = dmin(a, x);
          b = dmax(b, lo);
          a = hi;
        }
        wave_top2(a, b);
        if (lane == g) my_gs = (per == 1) ? a : a + b;
      }
      uint64_t kept = 0;
      for (int r = 0; r < p.topk_group; ++r) {
        const bool live = lane < p.G && !((kept >> lane) & 1ull);
        double v = live ? my_gs : NEG;
        int gi = live ? lane : 0x7FFFFFFF;
        wave_argbest(v, gi);
        kept |= 1ull << gi;
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        if (!((kept >> (e / per)) & 1ull)) c[i] = NEG;
      }
    }
  }

  // top-k among the open experts, in rank order.  Each lane first orders its
  // own candidates (value descending, then expert ascending: the swaps are
  // strict, so equal values keep the ascending order); a round then takes
  // the largest head over the lanes, and the lowest lane holding it holds
  // the lowest expert with that value (lane l holds experts l*EPL ..
  // l*EPL+EPL-1), which pops its head.  Lane j keeps rank j's expert and
  // selection score.
  uint64_t hk[EPL];
  double hs[EPL];
  int hx[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    hk[i] = order_key(c[i]);
    hs[i] = sv[i];
    hx[i] = lane * EPL + i;
  }
#pragma unroll
  for (int a = 1; a < EPL; ++a) {
#pragma unroll
    for (int b = a; b > 0; --b) {
      const bool sw = hk[b] > hk[b - 1];
      const uint64_t k0 = hk[b - 1];
      const double s0 = hs[b - 1];
      const int x0 = hx[b - 1];
      hk[b - 1] = sw ? hk[b] : k0;
      hs[b - 1] = sw ? hs[b] : s0;
      hx[b - 1] = sw ? hx[b] : x0;
      hk[b] = sw ? k0 : hk[b];
      hs[b] = sw ? s0 : hs[b];
      hx[b] = sw ? x0 : hx[b];
    }
  }
  int my_idx = 0;
  double my_raw = 0.0;
  for (int j = 0; j < p.K; ++j) {
    const uint64_t b = wave_max_key_lanes(hk[0]);
    const int owner = (int)__builtin_ctzll(b);
    const int ri = __builtin_amdgcn_readlane(hx[0], owner);
    const double s_win = readlane_d(hs[0], owner);
    if (lane == owner) {
#pragma unroll
      for (int i = 0; i + 1 < EPL; ++i) {
        hk[i] = hk[i + 1];
        hs[i] = hs[i + 1];
        hx[i] = hx[i + 1];
      }
      hk[EPL - 1] = 0;   // below every key of a finite or -inf value
    }
    my_idx = lane == j ? ri : my_idx;
    my_raw = lane == j ? s_win : my_raw;
  }
  // masses in rank order: the sigmoid values, or exp(z - z_max) for softmax
  // (every lane its own rank's), summed sequentially in rank order; lane j
  // keeps rank j's mass and the mass of the ranks before it (adaptive top-p)
  double contrib;
  if constexpr (SOFTMAX) {
    const double z0 = readlane_d(my_raw, 0);
    contrib = exp((lane < p.K ? my_raw : z0) - z0);
  } else {
    contrib = my_raw;
  }
  double ssum = 0.0, my_before = 0.0;
  for (int j = 0; j < p.K; ++j) {
    const double cj = readlane_d(contrib, j);
    my_before = lane == j ? ssum : my_before;
    ssum += cj;
  }
  const double my_s = contrib;
  // adaptive top-p: rank j stays when the mass before it is below top_p of
  // the total; the kept prefix's mass (the mass before the first dropped
  // rank) renormalizes the weights
  bool keep = true;
  double kept_sum = ssum;
  if (p.top_p > 0.0 && p.top_p < 1.0) {
    const double thr = p.top_p * ssum;
    keep = my_before < thr;
    const uint64_t kb = __ballot(lane < p.K && keep);
    const int m = __popcll(kb);   // a prefix: the masses are nonnegative
    if (m < p.K) kept_sum = readlane_d(my_before, m);
  }
  if (lane < p.K) {
    idx_out[lane] = keep ? my_idx : -1;
    w_out[lane] = keep ? (float)(my_s / kept_sum * (double)p.scaling) : 0.0f;
    if (idx_lds) idx_lds[lane] = keep ? my_idx : -1;
  }
}

// Selection for one token by one wave: zt = the token's E logits (or sct its
// scores); select_load then select_from.
template <int EPL, bool SOFTMAX>
__device__ __forceinline__ void select_token(const SelectParams& p, const double* __restrict__ zt,
                                             const float* __restrict__ bias, int32_t* idx_out,
                                             float* w_out, int32_t* idx_lds,
                                             const double* sct = nullptr) {
  double ra[EPL], rb[EPL];
  select_load<EPL, SOFTMAX>(p, zt, bias, sct, ra, rb);
  select_from<EPL, SOFTMAX>(p, sct != nullptr, ra, rb, idx_out, w_out, idx_lds);
}

// -------------------------------------------------------------- grouping
// Batch-union grouping ("colibri" README, "What's implemented"): a stable
// counting sort of the flat slots f = t*k + j by expert, in one block of
// BK_THREADS threads.  idx may point to global memory or to LDS.

constexpr int BK_THREADS = 1024;
constexpr int BK_WAVES = BK_THREADS / kWave;
constexpr int BK_KEY_BITS = 10;   // experts < 1024
constexpr int BK_SMALL = 512;     // slot counts up to this take the direct path
constexpr int BK_PER = 16;        // slots per thread read ahead by the general path
constexpr int64_t BK_CHUNK = (int64_t)BK_THREADS * BK_PER;

// LDS scratch of bucket_small (16-byte aligned).
struct __attribute__((aligned(16))) BucketSmallLds {
  int key[BK_SMALL];   // expert of the slot or -1 (invalid index, or padding to a multiple of 4)
  int kf[BK_SMALL];    // 2 * key + (first slot of its expert), or -1
  int rank[BK_SMALL];
  int off[kMaxExperts];
  int cnt[kMaxExperts];
  int before[kMaxExperts];   // index of the expert in the active list
  int n_active, n_valid;
};

// Small slot counts (F <= BK_SMALL): a slot's position is (slots of smaller
// experts) + (earlier slots of the same expert); every expert counts its
// slots itself, scanning the slot keys four at a time.  Any block size.
__device__ __forceinline__ void bucket_small(int32_t T, int32_t K, int32_t E, const int32_t* idx,
                                             int32_t* __restrict__ counts,
                                             int32_t* __restrict__ offsets,
                                             int32_t* __restrict__ entries,
                                             int32_t* __restrict__ inverse,
                                             int32_t* __restrict__ active,
                                             int32_t* __restrict__ n_active, BucketSmallLds& L,
                                             const SlotTables& tb = SlotTables{}) {
  int* s_key = L.key;
  int* s_kf = L.kf;
  int* s_rank = L.rank;
  int* s_off = L.off;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int F = T * K, F4 = (F + 3) & ~3;
  for (int f = tid; f < F4; f += nth) {
    const int e = f < F ? idx[f] : -1;
    s_key[f] = (e >= 0 && e < E) ? e : -1;
  }
  __syncthreads();
  for (int f = tid; f < F4; f += nth) {
    const int key = s_key[f];
    int r = 0;
    for (int g = 0; g < f; g += 4) {
      const int4 k4 = *reinterpret_cast<const int4*>(s_key + g);
      r += (k4.x == key) + (g + 1 < f && k4.y == key) + (g + 2 < f && k4.z == key) +
           (g + 3 < f && k4.w == key);
    }
    s_rank[f] = r;
    s_kf[f] = key < 0 ? -1 : 2 * key + (r == 0 ? 1 : 0);
  }
  __syncthreads();
  for (int e = tid; e < E; e += nth) {
    int off = 0, cnt = 0, before = 0;
#pragma unroll 4
    for (int g = 0; g < F4; g += 4) {
      const int4 v = *reinterpret_cast<const int4*>(s_kf + g);
      const int kf[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool lt = kf[q] >= 0 && kf[q] < 2 * e;
        off += lt ? 1 : 0;
        cnt += (kf[q] >> 1) == e ? 1 : 0;
        before += (lt && (kf[q] & 1)) ? 1 : 0;
      }
    }
    counts[e] = cnt;
    offsets[e] = off;
    s_off[e] = off;
    L.cnt[e] = cnt;
    L.before[e] = before;
    if (cnt) {
      active[before] = e;
      if (tb.slot_tab && before < tb.n_tab) {
        int32_t* r = tb.slot_tab + (int64_t)before * kSlotRec;
        r[0] = e;
        r[1] = off;
        r[2] = cnt;
      }
    }
    if (e == E - 1) {
      offsets[E] = off + cnt;
      n_active[0] = before + (cnt ? 1 : 0);
      L.n_active = before + (cnt ? 1 : 0);
      L.n_valid = off + cnt;
    }
  }
  __syncthreads();
  for (int f = tid; f < F; f += nth) {
    const int key = s_key[f];
    const int r = s_rank[f];
    const int pos = key < 0 ? -1 : s_off[key] + r;
    if (key >= 0) entries[pos] = f;
    inverse[f] = pos;   // -1 for a dropped slot
    if (key >= 0) {
      if (tb.pos_e) tb.pos_e[pos] = key;
      const int b = L.before[key];
      if (tb.slot_tab && b < tb.n_tab && r < 2) {
        int32_t* rec = tb.slot_tab + (int64_t)b * kSlotRec;
        rec[3 + r] = f;
        if (r == 0 && L.cnt[key] == 1) rec[4] = -1;
      }
    }
    // positions past the grouped slots (dropped ones) hold no expert
    if (tb.pos_e && f >= L.n_valid) tb.pos_e[f] = -1;
  }
  if (tb.slot_tab)
    for (int b = L.n_active + tid; b < tb.n_tab; b += nth) tb.slot_tab[(int64_t)b * kSlotRec] = -1;
}

__device__ void bucket_block(int32_t T, int32_t K, int32_t E, const int32_t* idx,
                             int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                             int32_t* __restrict__ entries, int32_t* __restrict__ inverse,
                             int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_wcnt[BK_WAVES][kMaxExperts];
  __shared__ int s_scan[BK_THREADS];
  __shared__ int s_flag[BK_THREADS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t F = (int64_t)T * K;

  // General path: LDS histogram, exclusive scan, scatter in rounds.
  for (int e = tid; e < E; e += BK_THREADS) {
    s_cnt[e] = 0;
    for (int w = 0; w < BK_WAVES; ++w) s_wcnt[w][e] = 0;
  }
  __syncthreads();
  // the slots are read in chunks of BK_PER per thread, all loads of a chunk
  // in flight together (the rounds below take them from registers)
  for (int64_t c0 = 0; c0 < F; c0 += BK_CHUNK) {
    int ev[BK_PER];
#pragma unroll
    for (int i = 0; i < BK_PER; ++i) {
      const int64_t f = c0 + (int64_t)i * BK_THREADS + tid;
      ev[i] = f < F ? idx[f] : -1;
    }
#pragma unroll
    for (int i = 0; i < BK_PER; ++i)
      if (ev[i] >= 0 && ev[i] < E) atomicAdd(&s_cnt[ev[i]], 1);
  }
  __syncthreads();

  // exclusive scans of the counts and of the nonzero flags (E <= 1024 = one
  // element per thread), Hillis-Steele in LDS
  const int v = tid < E ? s_cnt[tid] : 0;
  const int fl = v > 0 ? 1 : 0;
  s_scan[tid] = v;
  s_flag[tid] = fl;
  __syncthreads();
  for (int d = 1; d < BK_THREADS; d <<= 1) {
    const int a = tid >= d ? s_scan[tid - d] : 0;
    const int b = tid >= d ? s_flag[tid - d] : 0;
    __syncthreads();
    s_scan[tid] += a;
    s_flag[tid] += b;
    __syncthreads();
  }
  if (tid < E) {
    const int excl = s_scan[tid] - v;
    counts[tid] = v;
    offsets[tid] = excl;
    s_base[tid] = excl;
    if (fl) active[s_flag[tid] - 1] = tid;
  }
  if (tid == 0) {
    offsets[E] = s_scan[E - 1];
    n_active[0] = s_flag[E - 1];
  }
  __syncthreads();

  // Within a round of BK_THREADS slots, a slot's rank among equal experts
  // comes from ten ballots over the expert id's bits (the mask of lanes with
  // the same expert) and per-wave counts in LDS for earlier waves: no atomics
  // on positions, so the order is the stable one.
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t c0 = 0; c0 < F; c0 += BK_CHUNK) {
    int ev[BK_PER];
#pragma unroll
    for (int i = 0; i < BK_PER; ++i) {
      const int64_t f = c0 + (int64_t)i * BK_THREADS + tid;
      ev[i] = f < F ? idx[f] : -1;
    }
#pragma unroll
    for (int i = 0; i < BK_PER; ++i) {
      const int64_t f = c0 + (int64_t)i * BK_THREADS + tid;
      if (c0 + (int64_t)i * BK_THREADS >= F) break;   // uniform: past the last round
      const int e = ev[i];
      const bool valid = e >= 0 && e < E;
      uint64_t m = __ballot(valid);
#pragma unroll
      for (int b = 0; b < BK_KEY_BITS; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t bm = __ballot(bit);
        m &= bit ? bm : ~bm;
      }
      const int rank = __popcll(m & lt_mask);
      const int cnt = __popcll(m);
      const bool leader = valid && rank == 0;
      if (leader) s_wcnt[wave][e] = cnt;
      __syncthreads();
      if (valid) {
        int pos = s_base[e] + rank;
        for (int w = 0; w < wave; ++w) pos += s_wcnt[w][e];
        entries[pos] = (int32_t)f;
        inverse[f] = pos;
      } else if (f < F) {
        inverse[f] = -1;   // a dropped slot
      }
      __syncthreads();
      if (leader) {
        atomicAdd(&s_base[e], cnt);
        s_wcnt[wave][e] = 0;
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------- decode routing
__device__ __forceinline__ float4 load_x4(const void* x, int act_bf16, int64_t off) {
  if (act_bf16) {
    uint2 b = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + off);
    return make_float4(bf16_bits_to_f32(b.x & 0xFFFFu), bf16_bits_to_f32(b.x >> 16),
                       bf16_bits_to_f32(b.y & 0xFFFFu), bf16_bits_to_f32(b.y >> 16));
  }
  return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
}

// Router logits of expert row e for T <= 16 tokens, by one block of 256
// threads; red: LDS scratch of kDecodeTokens * 256 doubles.  Each thread
// requests its whole slice of the row (up to LG_QT 16-byte quads per pass)
// before any arithmetic -- branch-free, with clamped addresses -- so a row
// costs one memory round trip; the tokens then come from L1/L2.  Partial sums
// are reduced in LDS along a fixed tree (deterministic fp64 order).  The
// blocks of a launch (one per expert) also share out the sliced copies of the
// activation rows that sr asks for.
constexpr int LG_QT = 8;
__device__ __forceinline__ void logits_row_block(const float* __restrict__ W,
                                                 const void* __restrict__ x, int act_bf16,
                                                 int32_t T, int32_t H, int32_t E,
                                                 double* __restrict__ z, const SliceReq& sr,
                                                 int e, double* red, double* zsc = nullptr,
                                                 const float* zbias = nullptr) {
  const int tid = threadIdx.x;
  {
    const int ab = act_bf16 ? 2 : 4;
    const int64_t pieces = (int64_t)H * ab / 16;
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
    for (int64_t p = (int64_t)e * 256 + tid; p < pieces; p += (int64_t)E * 256)
      for (int n = 0; n < T; ++n) {
        const int64_t row = (int64_t)n * H * ab;
        if (sr.dst_a && sr.epg_a > 0)
          slice_piece(xb + row, reinterpret_cast<uint8_t*>(sr.dst_a) + row, p, sr.epg_a, ab);
        if (sr.dst_b && sr.epg_b > 0)
          slice_piece(xb + row, reinterpret_cast<uint8_t*>(sr.dst_b) + row, p, sr.epg_b, ab);
      }
  }
  const float* wr = W + (int64_t)e * H;
  const int nq = H / 4;
  const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
  double acc[kDecodeTokens];
#pragma unroll
  for (int n = 0; n < kDecodeTokens; ++n) acc[n] = 0.0;
  for (int q0 = 0; q0 < nq; q0 += 256 * LG_QT) {
    float4 w[LG_QT];
#pragma unroll
    for (int i = 0; i < LG_QT; ++i) {
      const int q = q0 + tid + 256 * i;
      const float4 v = *reinterpret_cast<const float4*>(wr + 4 * (q < nq ? q : nq - 1));
      w[i] = q < nq ? v : zero4;
    }
    for (int n = 0; n < T; ++n) {
      double a = 0.0;
#pragma unroll
      for (int i = 0; i < LG_QT; ++i) {
        const int q = q0 + tid + 256 * i;
        float4 v = load_x4(x, act_bf16, (int64_t)n * H + 4 * (q < nq ? q : nq - 1));
        if (q >= nq) v = zero4;
        a = fma((double)w[i].x, (double)v.x, a);
        a = fma((double)w[i].y, (double)v.y, a);
        a = fma((double)w[i].z, (double)v.z, a);
        a = fma((double)w[i].w, (double)v.w, a);
      }
#pragma unroll
      for (int m = 0; m < kDecodeTokens; ++m)
        if (m == n) acc[m] += a;
    }
  }
#pragma unroll
  for (int n = 0; n < kDecodeTokens; ++n)
    if (n < T) red[n * 256 + tid] = acc[n];
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st)
      for (int n = 0; n < T; ++n) red[n * 256 + tid] += red[n * 256 + tid + st];
    __syncthreads();
  }
  if (tid < T) {
    const double zv = red[tid * 256];
    z[(int64_t)tid * E + e] = zv;
    if (zsc) {
      // the sigmoid router's scores, as select_token forms them
      const double s = 1.0 / (1.0 + exp(-zv));
      zsc[((int64_t)tid * E + e) * 2] = s;
      zsc[((int64_t)tid * E + e) * 2 + 1] = s + (zbias ? (double)zbias[e] : 0.0);
    }
  }
}

// The grouping of one token's k slots (the result bucket_small gives for
// T = 1), by one wave with lane reads and no block barrier: the slots hold
// distinct experts (or -1, dropped), so slot j's bucket position is the
// number of kept slots with a smaller expert, every active expert has one
// row, and a kept expert's place in the active list is its position.  idx:
// the k expert indices (read by lanes < k, k <= 64); experts e = lane + 64 q
// (q < EPE) cover all E.
template <int EPE>
__device__ __forceinline__ void bucket_one_token(int32_t K, int32_t E, const int32_t* idx,
                                                 int32_t* __restrict__ counts,
                                                 int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ entries,
                                                 int32_t* __restrict__ inverse,
                                                 int32_t* __restrict__ active,
                                                 int32_t* __restrict__ n_active,
                                                 const SlotTables& tb) {
  const int lane = threadIdx.x & 63;
  const int e0 = lane < K ? idx[lane] : -1;
  const int key = (e0 >= 0 && e0 < E) ? e0 : -1;
  const int nval = __popcll(__ballot(key >= 0));
  int pos = 0, off[EPE], cnt[EPE];
#pragma unroll
  for (int q = 0; q < EPE; ++q) off[q] = cnt[q] = 0;
  for (int i = 0; i < K; ++i) {
    const int ki = __builtin_amdgcn_readlane(key, i);
    if (ki < 0) continue;   // wave-uniform
    pos += ki < key ? 1 : 0;
#pragma unroll
    for (int q = 0; q < EPE; ++q) {
      const int e = lane + 64 * q;
      off[q] += ki < e ? 1 : 0;
      cnt[q] += ki == e ? 1 : 0;
    }
  }
#pragma unroll
  for (int q = 0; q < EPE; ++q) {
    const int e = lane + 64 * q;
    if (e < E) {
      counts[e] = cnt[q];
      offsets[e] = off[q];
    }
  }
  if (lane == 0) {
    offsets[E] = nval;
    n_active[0] = nval;
  }
  if (lane < K) {
    inverse[lane] = key >= 0 ? pos : -1;
    if (key >= 0) {
      entries[pos] = lane;   // flat slot t * K + j of token 0
      active[pos] = key;
      if (tb.pos_e) tb.pos_e[pos] = key;
      if (tb.slot_tab && pos < tb.n_tab) {
        int32_t* r = tb.slot_tab + (int64_t)pos * kSlotRec;
        r[0] = key;
        r[1] = pos;
        r[2] = 1;
        r[3] = lane;
        r[4] = -1;
      }
    }
    // positions past the grouped slots hold no expert, nor records past the
    // active experts
    if (tb.pos_e && lane >= nval) tb.pos_e[lane] = -1;
    if (tb.slot_tab && lane >= nval && lane < tb.n_tab) tb.slot_tab[(int64_t)lane * kSlotRec] = -1;
  }
}

// LDS scratch of select_bucket_block.
struct __attribute__((aligned(16))) SelectBucketLds {
  BucketSmallLds b;
  int32_t idx[kDecodeTokens * kMaxTopK];
};

// Selection of all T <= 16 tokens (one wave each) and the grouping of their
// slots, by one block of 256 threads.  SIGMOID_ONLY: p is a sigmoid router
// (the softmax variant is not compiled in).
template <int EPL, bool SIGMOID_ONLY = false>
__device__ __forceinline__ void select_bucket_block(
    const SelectParams& p, const double* __restrict__ z, const float* __restrict__ bias,
    int32_t T, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ entries,
    int32_t* __restrict__ inverse, int32_t* __restrict__ active, int32_t* __restrict__ n_active,
    SelectBucketLds& L, const SlotTables& tb = SlotTables{}) {
  const int nw = blockDim.x >> 6;
  for (int t = threadIdx.x >> 6; t < T; t += nw) {
    if (!SIGMOID_ONLY && p.softmax)
      select_token<EPL, true>(p, z + (int64_t)t * p.E, bias, topk_idx + (int64_t)t * p.K,
                              topk_w + (int64_t)t * p.K, L.idx + t * p.K);
    else
      select_token<EPL, false>(p, z + (int64_t)t * p.E, bias, topk_idx + (int64_t)t * p.K,
                               topk_w + (int64_t)t * p.K, L.idx + t * p.K,
                               p.zsc ? p.zsc + (int64_t)t * p.E * 2 : nullptr);
  }
  __syncthreads();
  bucket_small(T, p.K, p.E, L.idx, counts, offsets, entries, inverse, active, n_active, L.b, tb);
}

}  // namespace moe
