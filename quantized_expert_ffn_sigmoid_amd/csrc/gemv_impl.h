// gemv_impl.h -- dequant-on-use expert GEMV for decode-sized buckets (gfx950).
//
// Experts are SwiGLU FFNs whose weights are packed int4 / packed int2 codes
// with one fp32 scale per output row, or bf16 ("colibri" README, "What's
// implemented": quantization kernels, per-row scales, dequant-on-use;
// "iliria" README, "What's implemented": routed-expert SwiGLU with gate and up
// over one activation).  Decode work is HBM-bound: every code byte is read
// once, so these kernels are organised around coalesced loads, enough bytes
// in flight, and a short unpack -- not around matrix cores.
//
// Work decomposition.  A matrix row is cut into granules of 16 bytes (8 for
// int2); the lpr lanes of a lane group (64, or fewer for short rows) share a
// row, lane j taking granules j, j + lpr, j + 2 lpr, ...  so that each load
// instruction of a wave reads whole 1 KB runs.  A lane keeps the activation
// values of its granule positions (its K-slice, KSL = K / lpr elements) in
// registers for the whole block, and the block's waves stream disjoint rows
// of one matrix (row pairs gate/up for the gate/up kernel) with several steps
// of loads in flight.  A row's partial dot products are summed over its lane
// group with DPP moves; the epilogue applies the per-row scale (constant along
// a row, so it commutes with the K-sum), SwiGLU, and writes h or y.
//
// Codes are unpacked as offset-binary bytes: an XOR of the sign bits, two
// masks, then packed conversions of byte pairs; the offset times the
// activation sum of the granule is removed once per granule.  Accumulation is
// fp32 throughout.
#pragma once

#include "moe_internal.h"
#include "route_device.h"
#include "unpack.h"

namespace moe {

template <int WDT>
struct Fmt;
// EPG: elements per granule, GB: granule bytes, DW: granule dwords.  The int
// formats unpack a code c (offset-binary, c = q + OFF) to c * UNIT: a byte
// 0..15 read as an OCP e4m3 float is exactly b * 2^-9 (subnormals, then the
// first binade), so one packed conversion yields two codes.
template <>
struct Fmt<MOE_I4> {
  static constexpr int EPG = 32, GB = 16, DW = 4;
  static constexpr float OFF = 8.0f, UNIT = 1.0f / 512.0f;
};
template <>
struct Fmt<MOE_I2> {
  static constexpr int EPG = 32, GB = 8, DW = 2;
  static constexpr float OFF = 2.0f, UNIT = 1.0f / 512.0f;
};
// int8: 32 codes in two 16-byte halves; a code q is read as the float
// (q + OFF) * UNIT, the same operand the int4 format yields for q in
// [-8, 7], so that int4 codes widened to int8 give bit-identical results.
template <>
struct Fmt<MOE_I8> {
  static constexpr int EPG = 32, GB = 32, DW = 8;
  static constexpr float OFF = 8.0f, UNIT = 1.0f / 512.0f;
};
template <>
struct Fmt<MOE_BF16> {
  static constexpr int EPG = 8, GB = 16, DW = 4;
  static constexpr float OFF = 0.0f, UNIT = 1.0f;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Codes are streamed once: non-temporal loads keep them from displacing the
// activations and router weights in the caches.
template <int WDT>
__device__ __forceinline__ void load_granule(const uint8_t* p, uint32_t (&g)[Fmt<WDT>::DW]) {
  if constexpr (Fmt<WDT>::DW == 8) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 16));
    g[0] = v.x;
    g[1] = v.y;
    g[2] = v.z;
    g[3] = v.w;
    g[4] = w.x;
    g[5] = w.y;
    g[6] = w.z;
    g[7] = w.w;
  } else if constexpr (Fmt<WDT>::DW == 4) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    g[0] = v.x;
    g[1] = v.y;
    g[2] = v.z;
    g[3] = v.w;
  } else {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    g[0] = v.x;
    g[1] = v.y;
  }
}

// 16 int8 codes (four dwords, element order) dotted with x[n][e0 .. e0+15]:
// offset bytes b = q + 128 are read exactly as floats, and (q + 8) * UNIT is
// one exact fma -- for q in [-8, 7] the very operand the int4 format yields.
template <int NT, int KSL>
__device__ __forceinline__ void i8_half_fma(const uint32_t (&gr)[4], const float (&x)[NT][KSL],
                                            int e0, float (&acc)[NT]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float q = i8_unpack_f32(gr[d], b);
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = fmaf(q, x[n][e0 + 4 * d + b], acc[n]);
    }
  }
}

// One granule (the g-th of the lane's K-slice) dotted with NT activation
// slices: acc[n] += sum_c q'_c * x[n][g*EPG + c], where q' = code + OFF for the
// int formats (the offset is removed per row from the slice sums).
template <int WDT, int NT, int KSL>
__device__ __forceinline__ void granule_fma(const uint32_t (&gr)[Fmt<WDT>::DW],
                                            const float (&x)[NT][KSL], int g, float (&acc)[NT]) {
  constexpr int EPG = Fmt<WDT>::EPG;
  const int b0 = g * EPG;
  if constexpr (WDT == MOE_I4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // offset-binary codes: even ones in ql, odd ones in qh
      float ql[4], qh[4];
      i4_unpack_f32(gr[d], ql, qh);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          acc[n] = fmaf(ql[b], x[n][b0 + 8 * d + 2 * b], acc[n]);
          acc[n] = fmaf(qh[b], x[n][b0 + 8 * d + 2 * b + 1], acc[n]);
        }
      }
    }
  } else if constexpr (WDT == MOE_I8) {
    const uint32_t lo[4] = {gr[0], gr[1], gr[2], gr[3]};
    const uint32_t hi[4] = {gr[4], gr[5], gr[6], gr[7]};
    i8_half_fma<NT, KSL>(lo, x, b0, acc);
    i8_half_fma<NT, KSL>(hi, x, b0 + 16, acc);
  } else if constexpr (WDT == MOE_I2) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float q[4];
        i2_unpack_f32(gr[d], jj, q);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[n] = fmaf(q[b], x[n][b0 + 16 * d + 4 * b + jj], acc[n]);
        }
      }
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float q0 = __uint_as_float(gr[d] << 16);
      const float q1 = __uint_as_float(gr[d] & 0xFFFF0000u);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        acc[n] = fmaf(q0, x[n][b0 + 2 * d], acc[n]);
        acc[n] = fmaf(q1, x[n][b0 + 2 * d + 1], acc[n]);
      }
    }
  }
}

// A DPP lane move whose every source lane is valid (quad permutes, mirrors),
// written so that the compiler folds it into the add that consumes it.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// a + b over the lane pairs (l, l ^ 16) and (l, l ^ 32): the permlane swaps
// exchange 16-lane rows (odd rows of one copy with even rows of the other) and
// 32-lane halves, so the two results hold the pair's two values.
__device__ __forceinline__ float add_swap16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float add_swap32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Sum over aligned groups of lpr lanes (a power of two); every lane of a group
// receives the group's sum.  Quad swaps and the 8- and 16-lane mirrors are DPP
// operands of the adds; the 32- and 64-lane steps swap rows and halves between
// registers (no LDS round trip).  Each step adds lane l and its partner in the
// same pairs, and a + b = b + a, so all lanes hold the same bits.
__device__ __forceinline__ float group_sum(float v, int lpr) {
  if (lpr >= 2) v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  if (lpr >= 4) v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  if (lpr >= 8) v += dpp_f<0x141>(v);   // row_half_mirror
  if (lpr >= 16) v += dpp_f<0x140>(v);  // row_mirror
  if (lpr >= 32) v = add_swap16(v);
  if (lpr >= 64) v = add_swap32(v);
  return v;
}


// Activation slice of one row in registers: x[g*EPG + c] = row[(g*lpr + j)*EPG + c]
// for the lane's GPL granules; gsum[g] = the sum of granule g's values (for the
// int offset).  Rows are f32 or bf16 (widened exactly).
template <int EPG, int KSL, int ABF16>
__device__ __forceinline__ void load_slice(const void* base, int64_t row_off, int lpr, int j,
                                           float (&x)[KSL], float (&gsum)[KSL / EPG]) {
  constexpr int GPL = KSL / EPG;
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int64_t k0 = row_off + (int64_t)(g * lpr + j) * EPG;
    float s = 0.f;
    if constexpr (ABF16) {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + k0;
#pragma unroll
      for (int c = 0; c < EPG; c += 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(p + c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          x[g * EPG + c + 2 * d] = __uint_as_float(w[d] << 16);
          x[g * EPG + c + 2 * d + 1] = __uint_as_float(w[d] & 0xFFFF0000u);
          s += x[g * EPG + c + 2 * d] + x[g * EPG + c + 2 * d + 1];
        }
      }
    } else {
      const float* p = reinterpret_cast<const float*>(base) + k0;
#pragma unroll
      for (int c = 0; c < EPG; c += 4) {
        const float4 v = *reinterpret_cast<const float4*>(p + c);
        x[g * EPG + c] = v.x;
        x[g * EPG + c + 1] = v.y;
        x[g * EPG + c + 2] = v.z;
        x[g * EPG + c + 3] = v.w;
        s += (v.x + v.y) + (v.z + v.w);
      }
    }
    gsum[g] = s;
  }
}

// ------------------------------------------------------------ block jobs
// A block of kWaves waves owns rows [r0, r0 + nr) of one matrix; wave w
// takes passes w, w + kWaves, ...  A pass covers rpp rows (one per lane group
// of lpr lanes).  The codes of the next PF passes are in flight while one is
// computed; activation slices stay in registers for the whole block.

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

// Pipelining step: CG granules of each of the NM rows of a pass (a row's GPL
// granules take GPL / CG steps).  A step holds at most 96 bytes per lane (six
// 16-byte or three 32-byte granules; 8-byte granules count as 16); PF steps
// are in flight while one is computed.
template <int GPL, int NM, int GB>
struct StepShape {
  static constexpr int kMaxG = GB > 16 ? 3 : 6;
  static constexpr int cg_for(int c) { return (GPL % c == 0 && c * NM <= kMaxG) ? c : cg_for(c - 1); }
  static constexpr int CG = cg_for(GPL < 6 ? GPL : 6);
  static constexpr int STEPS = GPL / CG;
  static constexpr int PF = CG * NM >= 4 ? 2 : (CG * NM >= 2 ? 4 : 8);
};

struct Job {
  const uint8_t* W;    // matrix [rows][K] of this expert
  const float* S;      // per-row scales (unused for bf16)
  int K, rows;         // input length, output rows (gate/up: row pairs)
  int lpr, rpp;        // lanes per row, rows per pass
  int r0, nr;          // the block's rows
};

// nt (<= NT) activation rows at element offsets xoff[] through the block's
// rows.  PAIR: gate row r and up row r + rows, combined by SwiGLU into
// h[hrow[n]][r]; otherwise y[yrow[n]][r] = scaled dot.
template <int WDT, int KSL, int NT, int ABF16, bool PAIR>
__device__ void job_chunk(const Job& jb, const void* src, const int64_t* xoff, int nt,
                          void* dst, const int64_t* drow, float* probe) {
  using F = Fmt<WDT>;
  constexpr int EPG = F::EPG, GB = F::GB, DW = F::DW, GPL = KSL / EPG;
  constexpr int NM = PAIR ? 2 : 1;
  using SS = StepShape<GPL, NM, GB>;
  constexpr int CG = SS::CG, STEPS = SS::STEPS, PF = SS::PF;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lpr = jb.lpr, rpp = jb.rpp;
  const int j = lane & (lpr - 1), rg = lane / lpr;
  const int64_t rbytes = (int64_t)(jb.K / EPG) * GB;

  float x[NT][KSL], gs[NT][GPL];
#pragma unroll
  for (int n = 0; n < NT; ++n) load_slice<EPG, KSL, ABF16>(src, xoff[n < nt ? n : 0], lpr, j, x[n], gs[n]);

  const int passes = (jb.nr + rpp - 1) / rpp;
  const int mine = wave < passes ? (passes - wave + kWaves - 1) / kWaves : 0;
  const int nsteps = mine * STEPS;
  auto row_of = [&](int i, bool& ok) {
    const int rl = (wave + i * kWaves) * rpp + rg;
    const int r = jb.r0 + rl;
    ok = rl < jb.nr && r < jb.rows;
    return ok ? r : jb.r0;
  };
  // step t = pass t / STEPS, granules [(t % STEPS) * CG, +CG) of each row;
  // the last step of a row also fetches the row scales, so that no load sits
  // on the epilogue's path
  auto load_step = [&](int t, uint32_t (&b)[NM][CG][DW], float (&sc)[NM]) {
    bool ok;
    const int r = row_of(t / STEPS, ok);
    const int g0 = (t % STEPS) * CG;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint8_t* rp = jb.W + (int64_t)(r + m * jb.rows) * rbytes;
#pragma unroll
      for (int g = 0; g < CG; ++g)
        load_granule<WDT>(rp + (int64_t)((g0 + g) * lpr + j) * GB, b[m][g]);
      if constexpr (WDT != MOE_BF16)
        if (t % STEPS == STEPS - 1) sc[m] = jb.S[r + m * jb.rows];
    }
  };

  uint32_t buf[PF][NM][CG][DW];
  float sbuf[PF][NM];
#pragma unroll
  for (int k = 0; k < PF; ++k)
    if (k < nsteps) load_step(k, buf[k], sbuf[k]);

  float acc[NM][NT];
  for (int base = 0; base < nsteps; base += PF) {
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      const int t = base + k;
      if (t < nsteps) {
        const int sc = t % STEPS;
        if (sc == 0) {
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[m][n] = 0.f;
        }
        // the step's granules: compile-time positions within the slice for
        // each possible sc (STEPS is small), selected by a uniform branch
#pragma unroll
        for (int s2 = 0; s2 < STEPS; ++s2) {
          if (s2 == sc) {
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
              for (int g = 0; g < CG; ++g) {
                granule_fma<WDT, NT, KSL>(buf[k][m][g], x, s2 * CG + g, acc[m]);
                if constexpr (WDT != MOE_BF16) {
#pragma unroll
                  for (int n = 0; n < NT; ++n)
                    acc[m][n] = fmaf(-F::OFF * F::UNIT, gs[n][s2 * CG + g], acc[m][n]);
                }
              }
          }
        }
        float scale[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) scale[m] = sbuf[k][m];
        if (t + PF < nsteps) load_step(t + PF, buf[k], sbuf[k]);
        if (sc == STEPS - 1) {
          bool ok;
          const int r = row_of(t / STEPS, ok);
          float red[NM][NT];
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int n = 0; n < NT; ++n) red[m][n] = group_sum(acc[m][n], lpr);
          if (ok) {
            float sa = 1.f, sb = 1.f;
            if constexpr (WDT != MOE_BF16) {
              sa = scale[0] * (1.0f / F::UNIT);
              if constexpr (PAIR) sb = scale[NM - 1] * (1.0f / F::UNIT);
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) {
              if (n < nt && j == (n & (lpr - 1))) {
                if constexpr (PAIR) {
                  const float gv = red[0][n] * sa, uv = red[1][n] * sb;
                  const float hv = gv / (1.0f + expf(-gv)) * uv;
                  if constexpr (ABF16)
                    reinterpret_cast<uint16_t*>(dst)[drow[n] * jb.rows + r] = f32_to_bf16_bits(hv);
                  else
                    reinterpret_cast<float*>(dst)[drow[n] * jb.rows + r] = hv;
                  if (probe) probe[drow[n] * jb.rows + r] = hv;
                } else {
                  reinterpret_cast<float*>(dst)[drow[n] * jb.rows + r] = red[0][n] * sa;
                }
              }
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------ ring path
// Rows of at least 64 granules (all 64 lanes of a wave on one row, so every
// wave load is one contiguous 1 KB run; int8's 32-byte granules take two
// slots, each a 2 KB run read at every other 16 bytes; int2's 8-byte granules
// go two 512-byte granule runs to a slot, lanes 0-31 loading the first and
// lanes 32-63 the second, one load instruction per slot as for the other
// formats): the codes stream through a per-wave
// ring of kRing 1 KB LDS slots filled by direct global-to-LDS loads.  Loads
// in flight then hold no registers, and a slot is refilled as soon as its
// data has been consumed, so about kRing KB per wave stay in flight.
// Completion is tracked with explicit vmcnt waits.  Inside the loop the only
// vector memory instructions are the ring loads (row results go to LDS and
// are written at the end of the block; row scales are staged in LDS first),
// and loads complete in issue order, so "slot n has landed" is "no more than
// the number of younger ring loads are pending".
constexpr int kRing = 16;
constexpr int kMaxRingRows = 512;   // rows per block on the ring path

struct __attribute__((aligned(16))) RingLds {
  uint8_t ring[kWaves][kRing][1024];
  float out[2][kMaxRingRows];     // per token of the chunk
  float scale[2][kMaxRingRows];   // gate (or the only matrix), up
};

// Waits until at most N vector memory loads are outstanding.  The asm form
// keeps memory accesses from moving across the wait; the builtin repeats it
// in a form the compiler's own wait insertion sees, so that it does not wait
// again (for everything) before using registers loaded earlier.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  // gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 at
  // their maxima (no wait)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Activation slices through LDS: the block copies the nt activation rows into
// LDS with coalesced 16-byte loads (all blocks read the same few rows, so
// per-lane strided loads would flood the L2 with requests), then every lane
// reads its granules' activations.  Chunk q -- the EPG activations of granule
// q -- sits at q * (CB + 16) bytes; the padding puts the 16-byte reads of 16
// consecutive lanes on distinct banks.  Ends with a barrier, after which the
// staging area may be reused.
template <int EPG, int KSL, int NT, int ABF16>
__device__ __forceinline__ void slices_via_lds(const void* src, const int64_t* xoff, int nt, int K,
                                               uint8_t* stage, float (&x)[NT][KSL],
                                               float (&gs)[NT][KSL / EPG]) {
  constexpr int AB = ABF16 ? 2 : 4, CB = EPG * AB, CS = CB + 16, PPC = CB / 16;
  constexpr int GPL = KSL / EPG;
  static_assert(NT * (KSL * 64 / EPG) * CS <= kWaves * kRing * 1024, "staging fits the ring area");
  const int rowb = (K / EPG) * CS;
  const int pieces = K * AB / 16;
  for (int n = 0; n < nt && n < NT; ++n) {
    const uint8_t* g = reinterpret_cast<const uint8_t*>(src) + xoff[n] * AB;
    for (int p = threadIdx.x; p < pieces; p += kThreads) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(g + (int64_t)p * 16);
      const int q = p / PPC, r = p - q * PPC;
      *reinterpret_cast<u32x4*>(stage + n * rowb + q * CS + r * 16) = v;
    }
  }
  __syncthreads();
  const int j = threadIdx.x & 63;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const uint8_t* row = stage + (n < nt ? n : 0) * rowb;
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const uint8_t* c = row + (g * 64 + j) * CS;
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < PPC; ++r) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(c + r * 16);
        if constexpr (ABF16) {
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const float lo = __uint_as_float(w[d] << 16), hi = __uint_as_float(w[d] & 0xFFFF0000u);
            x[n][g * EPG + r * 8 + 2 * d] = lo;
            x[n][g * EPG + r * 8 + 2 * d + 1] = hi;
            s += lo + hi;
          }
        } else {
          const float f[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                              __uint_as_float(v.w)};
#pragma unroll
          for (int d = 0; d < 4; ++d) x[n][g * EPG + r * 4 + d] = f[d];
          s += (f[0] + f[1]) + (f[2] + f[3]);
        }
      }
      gs[n][g] = s;
    }
  }
  __syncthreads();
}

// Activation slices read straight from rows in the sliced layout: lane j's
// piece c of granule g is the 16 bytes at ((g * PPC + c) * 64 + j) * 16, so
// every load instruction of the wave reads one contiguous 1 KB run.
// The loads only (bf16 rows stay packed in x's registers until
// slice_finish), so that the caller can issue more loads before the first
// use of these.
template <int EPG, int KSL, int NT, int ABF16>
__device__ __forceinline__ void slices_sliced_load(const void* src, const int64_t* xoff, int nt,
                                                   float (&x)[NT][KSL]) {
  constexpr int AB = ABF16 ? 2 : 4, P = 16 / AB, PPC = EPG / P, GPL = KSL / EPG;
  const int j = threadIdx.x & 63;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const uint8_t* row = reinterpret_cast<const uint8_t*>(src) + xoff[n < nt ? n : 0] * AB;
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
#pragma unroll
      for (int c = 0; c < PPC; ++c) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row + ((int64_t)(g * PPC + c) * 64 + j) * 16);
        // 16 bytes: 4 floats, or 8 bf16 kept in the first 4 slots of the piece
        const int b = ABF16 ? g * EPG + c * 8 : g * EPG + c * 4;
        x[n][b] = __uint_as_float(v.x);
        x[n][b + 1] = __uint_as_float(v.y);
        x[n][b + 2] = __uint_as_float(v.z);
        x[n][b + 3] = __uint_as_float(v.w);
      }
    }
  }
}

// Activation slices read from rows in natural order: lane j's piece c of
// granule g is the 16 bytes at ((g * 64 + j) * PPC + c) * 16, so one load
// instruction of the wave spans the 64 granules of one row segment (every
// wave of a block reads the whole row; it stays in the caches).  The loads
// only, with the register layout of slices_sliced_load.
template <int EPG, int KSL, int NT, int ABF16>
__device__ __forceinline__ void slices_natural_load(const void* src, const int64_t* xoff, int nt,
                                                    float (&x)[NT][KSL]) {
  constexpr int AB = ABF16 ? 2 : 4, P = 16 / AB, PPC = EPG / P, GPL = KSL / EPG;
  const int j = threadIdx.x & 63;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const uint8_t* row = reinterpret_cast<const uint8_t*>(src) + xoff[n < nt ? n : 0] * AB;
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
#pragma unroll
      for (int c = 0; c < PPC; ++c) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row + ((int64_t)(g * 64 + j) * PPC + c) * 16);
        const int b = ABF16 ? g * EPG + c * 8 : g * EPG + c * 4;
        x[n][b] = __uint_as_float(v.x);
        x[n][b + 1] = __uint_as_float(v.y);
        x[n][b + 2] = __uint_as_float(v.z);
        x[n][b + 3] = __uint_as_float(v.w);
      }
    }
  }
}

// Widens packed bf16 pieces (bf16 rows) and forms the granule sums.
template <int EPG, int KSL, int NT, int ABF16>
__device__ __forceinline__ void slice_finish(float (&x)[NT][KSL], float (&gs)[NT][KSL / EPG]) {
  constexpr int P = ABF16 ? 8 : 4, PPC = EPG / P, GPL = KSL / EPG;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < PPC; ++c) {
        if constexpr (ABF16) {
          const int b = g * EPG + c * 8;
          const uint32_t w[4] = {__float_as_uint(x[n][b]), __float_as_uint(x[n][b + 1]),
                                 __float_as_uint(x[n][b + 2]), __float_as_uint(x[n][b + 3])};
#pragma unroll
          for (int d = 3; d >= 0; --d) {
            const float lo = __uint_as_float(w[d] << 16), hi = __uint_as_float(w[d] & 0xFFFF0000u);
            x[n][b + 2 * d] = lo;
            x[n][b + 2 * d + 1] = hi;
          }
#pragma unroll
          for (int d = 0; d < 4; ++d) s += x[n][b + 2 * d] + x[n][b + 2 * d + 1];
        } else {
          const int b = g * EPG + c * 4;
          s += (x[n][b] + x[n][b + 1]) + (x[n][b + 2] + x[n][b + 3]);
        }
      }
      gs[n][g] = s;
    }
  }
}

// The wave's stream over its rows of a block: item t is local row
// i = t / S (rows wave, wave + kWaves, ...), matrix m, granule g, half h; ring
// slot n holds item n, or items 2n and 2n + 1 (int2).
template <int WDT, int KSL, bool PAIR>
struct RingStream {
  static constexpr int EPG = Fmt<WDT>::EPG, GB = Fmt<WDT>::GB, GPL = KSL / EPG;
  static constexpr int HPG = GB >= 16 ? GB / 16 : 1;   // 16-byte slots per granule: 1, or 2 (int8 halves)
  static constexpr int IPS = GB == 8 ? 2 : 1;          // items per slot
  static constexpr int NM = PAIR ? 2 : 1, S = NM * GPL * HPG;
  const uint8_t* lane_base;
  int64_t rbytes;
  int rows, wave, items, total;   // total: slots
  uint8_t* ring;

  __device__ __forceinline__ RingStream(const Job& jb, int nr, RingLds& L) {
    const int lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    rbytes = (int64_t)(jb.K / EPG) * GB;
    rows = jb.rows;
    const int my_rows = wave < nr ? (nr - wave + kWaves - 1) / kWaves : 0;
    items = my_rows * S;
    total = (items + IPS - 1) / IPS;
    ring = &L.ring[wave][0][0];
    lane_base = jb.W + (int64_t)jb.r0 * rbytes + (IPS == 2 ? (lane & 31) * 16 : lane * GB);
  }
  __device__ __forceinline__ const uint8_t* item_addr(int t) const {
    const int i = t / S, idx = t - i * S;
    const int m = idx / (GPL * HPG), gh = idx - m * (GPL * HPG);
    const int g = gh / HPG, h = gh - g * HPG;
    const int64_t row = wave + i * kWaves + m * rows;
    return lane_base + row * rbytes + g * (64 * GB) + h * 16;
  }
  __device__ __forceinline__ const uint8_t* slot_addr(int n) const {
    if constexpr (IPS == 1) {
      return item_addr(n);
    } else {
      // an odd item count leaves the last slot's second half reloading the
      // block's first granule run, never read
      const int t = 2 * n + ((threadIdx.x >> 5) & 1);
      return t < items ? item_addr(t) : lane_base;
    }
  }
  __device__ __forceinline__ void issue_at(const uint8_t* p, int n) const {
    // non-temporal: the codes are read once
    __builtin_amdgcn_global_load_lds(p, (lds_ptr_t)(ring + (n & (kRing - 1)) * 1024), 16, 0, 2);
  }
  __device__ __forceinline__ void issue(int n) const { issue_at(slot_addr(n), n); }
  // Slots [N0, N1) of the ring's first fill; slots past the stream reload the
  // block's first granule into ring slots that are never read, so that every
  // wave issues the same loads.
  template <int N0, int N1>
  __device__ __forceinline__ void prologue() const {
#pragma unroll
    for (int n = N0; n < N1; ++n) issue_at(n < total ? slot_addr(n) : lane_base, n);
  }
};

// Ring slots issued before the activation loads.  Register loads and direct
// LDS loads outstanding together make the compiler wait for all of them
// before the first use of a loaded register, so the activations are waited
// for once, early, with only these slots in flight; the rest of the first
// fill follows.
constexpr int kRingPre = 4;

// Row scales of a wave's rows (local rows wave, wave + kWaves, ...) into its
// part of L.scale by direct global-to-LDS loads: no register waits; the ring's
// first wait covers them, as they are issued before the ring's loads.
constexpr int kScalePerWave = kMaxRingRows / kWaves;
__device__ __forceinline__ float* wave_scales(RingLds& L, int m, int wave) {
  return &L.scale[m][wave * kScalePerWave];
}
template <bool PAIR>
__device__ __forceinline__ void stage_wave_scales(const Job& jb, int nr, int wave, RingLds& L) {
  const int lane = threadIdx.x & 63;
  const int my_rows = wave < nr ? (nr - wave + kWaves - 1) / kWaves : 0;
  for (int c = 0; c < my_rows; c += 64) {
    const int i = c + lane;
    const int r = jb.r0 + (i < my_rows ? wave + i * kWaves : 0);
#pragma unroll
    for (int m = 0; m < (PAIR ? 2 : 1); ++m)
      __builtin_amdgcn_global_load_lds(jb.S + m * jb.rows + r, (lds_ptr_t)(wave_scales(L, m, wave) + c),
                                       4, 0, 0);
  }
}

// The wave's rows of the block: local rows wave, wave + kWaves, ... < nr.
// Row results (scaled, SwiGLU applied for PAIR) go to L.out[n][local row].
// Activation rows are read sliced, or staged through the ring area before the
// ring starts, or (PRE) were read by the caller, who passes the slices and
// their granule sums in xpre / gpre: then the whole first fill is issued at
// once.  NATX (rows in natural order): the wave reads its slices with
// register loads, issues the whole first fill behind them and waits for the
// activations only.  Every wave of the block calls this together.
template <int WDT, int KSL, int NT, int ABF16, bool PAIR, bool SLICED, bool PRE = false,
          bool NATX = false>
__device__ __forceinline__ void job_ring(const Job& jb, int nr, const void* src, const int64_t* xoff,
                                         int nt, RingLds& L, const float* xpre = nullptr,
                                         const float* gpre = nullptr) {
  using F = Fmt<WDT>;
  using RS = RingStream<WDT, KSL, PAIR>;
  constexpr int EPG = F::EPG, GB = F::GB, GPL = KSL / EPG;
  constexpr int HPG = RS::HPG, NM = RS::NM, S = RS::S;
  static_assert(GB == 16 || (GB == 32 && WDT == MOE_I8) || (GB == 8 && WDT == MOE_I2),
                "ring slots hold 16-byte granules, halves of int8 ones or pairs of int2 ones");
  static_assert(WDT != MOE_I8 || (Fmt<MOE_I8>::UNIT == 1.0f / 512.0f && Fmt<MOE_I8>::OFF == 8.0f),
                "i8_half_fma's constants");
  static_assert(kMaxRingRows % kWaves == 0, "per-wave scale areas");
  const int lane = threadIdx.x & 63;

  constexpr int IPS = RS::IPS;
  const RS st(jb, nr, L);
  const int wave = st.wave, total = st.total, my_rows = st.items / S;
  uint8_t* ring = st.ring;
  // order of the loads: row scales and the first ring slots, the
  // activations (waited for at once), then the rest of the ring's first fill
  if constexpr (WDT != MOE_BF16) stage_wave_scales<PAIR>(jb, nr, wave, L);
  float x[NT][KSL], gs[NT][GPL];
  if constexpr (PRE) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int k = 0; k < KSL; ++k) x[n][k] = xpre[n * KSL + k];
#pragma unroll
      for (int g = 0; g < GPL; ++g) gs[n][g] = gpre[n * GPL + g];
    }
    st.template prologue<0, kRing>();
  } else if constexpr (NATX) {
    slices_natural_load<EPG, KSL, NT, ABF16>(src, xoff, nt, x);
    st.template prologue<0, kRing>();
    // the activation loads, issued before the ring's kRing, have landed
    wait_vmcnt<kRing>();
    slice_finish<EPG, KSL, NT, ABF16>(x, gs);
  } else if constexpr (!SLICED) {
    // the ring area stages the activation rows first
    slices_via_lds<EPG, KSL, NT, ABF16>(src, xoff, nt, jb.K, &L.ring[0][0][0], x, gs);
    st.template prologue<0, kRing>();
  } else {
    st.template prologue<0, kRingPre>();
    slices_sliced_load<EPG, KSL, NT, ABF16>(src, xoff, nt, x);
    slice_finish<EPG, KSL, NT, ABF16>(x, gs);
    // the granule sums are formed (so the activations have landed) before the
    // rest of the fill is issued
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int g = 0; g < GPL; ++g) asm volatile("" : "+v"(gs[n][g]) : : "memory");
    st.template prologue<kRingPre, kRing>();
  }
  const float* sc0 = wave_scales(L, 0, wave);
  const float* sc1 = wave_scales(L, PAIR ? 1 : 0, wave);

  auto read_item = [&](int t) {
    if constexpr (IPS == 1) {
      return *reinterpret_cast<const u32x4*>(ring + (t & (kRing - 1)) * 1024 + lane * 16);
    } else {
      const u32x2 v = *reinterpret_cast<const u32x2*>(ring + ((t >> 1) & (kRing - 1)) * 1024 +
                                                      (t & 1) * 512 + lane * 8);
      return u32x4{v.x, v.y, 0u, 0u};
    }
  };
  // item t + 1 is read while item t is computed; before the read of a slot's
  // first item, the loads younger than that slot are ring refills (and, early
  // on, the activation and scale loads, which only make the count
  // conservative), at most kRing - 2 of them
  u32x4 vnext = {0u, 0u, 0u, 0u};
  if (total > 0) {
    if (total - 1 >= kRing - 2) wait_vmcnt<kRing - 2>();
    else wait_vmcnt<0>();
    vnext = read_item(0);
  }

  for (int i = 0; i < my_rows; ++i) {
    float acc[NM][NT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[m][n] = 0.f;
#pragma unroll
    for (int idx = 0; idx < S; ++idx) {
      const int t = i * S + idx;
      const int sn = t / IPS;   // the item's slot
      const u32x4 v = vnext;
      if (t + 1 < st.items) {
        if ((t + 1) % IPS == 0) {
          if (total - sn - 2 >= kRing - 2) wait_vmcnt<kRing - 2>();
          else wait_vmcnt<0>();
        }
        vnext = read_item(t + 1);
      }
      const int mm = idx / (GPL * HPG), gh = idx % (GPL * HPG);
      const int g = gh / HPG, h = gh % HPG;
      if constexpr (IPS == 2) {
        const uint32_t gr[2] = {v.x, v.y};
        granule_fma<WDT, NT, KSL>(gr, x, g, acc[mm]);
      } else {
        const uint32_t gr[4] = {v.x, v.y, v.z, v.w};
        if constexpr (HPG == 1) granule_fma<WDT, NT, KSL>(gr, x, g, acc[mm]);
        else i8_half_fma<NT, KSL>(gr, x, g * EPG + 16 * h, acc[mm]);
      }
      if constexpr (WDT != MOE_BF16) {
        // the offset after the granule's last slot
        if (h == HPG - 1) {
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[mm][n] = fmaf(-F::OFF * F::UNIT, gs[n][g], acc[mm][n]);
        }
      }
      // after its last item the slot has been consumed (its data fed the
      // FMAs above): refill it
#pragma unroll
      for (int n = 0; n < NT; ++n) asm volatile("" : "+v"(acc[mm][n]) : "v"(v.x), "v"(IPS == 2 ? v.y : v.w) : "memory");
      if (t % IPS == IPS - 1 && sn + kRing < total) st.issue(sn + kRing);
    }
    const int rl = wave + i * kWaves;
    float red[NM][NT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) red[m][n] = group_sum(acc[m][n], 64);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (n < nt && lane == n) {
        float sa = 1.f, sb = 1.f;
        if constexpr (WDT != MOE_BF16) {
          sa = sc0[i] * (1.0f / F::UNIT);
          if constexpr (PAIR) sb = sc1[i] * (1.0f / F::UNIT);
        }
        if constexpr (PAIR) {
          const float gv = red[0][n] * sa, uv = red[1][n] * sb;
          L.out[n][rl] = gv / (1.0f + expf(-gv)) * uv;
        } else {
          L.out[n][rl] = red[0][n] * sa;
        }
      }
    }
  }
  // a wave with fewer rows than the first fill (or none) still has loads in
  // flight into its ring slots
  if (total < kRing) wait_vmcnt<0>();
}

// Which matrix and which token rows a block handles.  Routed and shared
// blocks are interleaved evenly over the grid, so that the CUs each get a mix
// of the two (their unpack costs per byte differ).
struct BlockWork {
  bool shared;
  bool have_f;   // f0, f1: flat slots of rows 0 and 1 (from the slot tables)
  int e, p0, nrows, rb_index;
  int f0, f1;    // scalars: an indexed array here would be placed in LDS
};

// Logical id of block b of n such that the blocks the hardware deals to one
// XCD (b mod 8) take consecutive logical ids.
__device__ __forceinline__ int64_t xcd_logical(int64_t b, int64_t n) {
  const int64_t q = n >> 3, r = n & 7, x = b & 7;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + (b >> 3);
}

// b: the block's index among the launch's GEMV blocks.
__device__ __forceinline__ bool block_work(const GemvArgs& a, BlockWork& bw, int64_t b) {
  const int64_t routed_blocks = (int64_t)a.n_slots * a.nb;
  const int64_t shared_blocks = (int64_t)a.nb_s * a.ntg_s;
  const int64_t nblk = routed_blocks + shared_blocks;
  // token mode: the blocks that read the same weight rows for different tokens
  // sit next to each other on one XCD, so the rows come from HBM once
  const int64_t bid = a.per_token ? xcd_logical(b, nblk) : b;
  bw.have_f = false;
  const int64_t before = bid * shared_blocks / nblk;       // shared blocks before bid
  const bool is_shared = (bid + 1) * shared_blocks / nblk > before;
  const RowSource& src = a.src;
  if (!is_shared) {
    const int64_t rbid = bid - before;
    bw.shared = false;
    if (a.per_token) {
      const int p = (int)(rbid % a.n_slots);
      bw.rb_index = (int)(rbid / a.n_slots);
      bw.p0 = p;
      bw.nrows = 1;
      if (src.routed && src.pos_e) {
        // the position's expert and flat slot, read together
        const int e = src.pos_e[p];
        const int f = src.entries[p];
        if (e < 0) return false;
        bw.e = e;
        bw.f0 = f;
        bw.f1 = -1;
        bw.have_f = true;
      } else if (src.routed) {
        // the active expert whose bucket holds position p (buckets are
        // contiguous and ascending with the active list)
        const int na = *src.n_active;
        if (na <= 0) return false;
        int lo = 0, hi = na - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (src.offsets[src.active[mid]] <= p) lo = mid; else hi = mid - 1;
        }
        bw.e = src.active[lo];
        if (p >= src.offsets[bw.e + 1]) return false;
      } else {
        bw.e = src.fixed_expert;
        if (p >= src.n_rows) return false;
      }
      return true;
    }
    const int slot = (int)(rbid / a.nb);
    bw.rb_index = (int)(rbid - (int64_t)slot * a.nb);
    if (src.routed && src.slot_tab) {
      // the slot's whole assignment in one read
      const int32_t* r = src.slot_tab + (int64_t)slot * kSlotRec;
      const int4 v = *reinterpret_cast<const int4*>(r);
      const int f1 = r[4];
      if (v.x < 0) return false;
      bw.e = v.x;
      bw.p0 = v.y;
      bw.nrows = v.z;
      bw.f0 = v.w;
      bw.f1 = f1;
      bw.have_f = true;
    } else if (src.routed) {
      // the active count and the slot's entry in one round trip (slot <
      // n_slots <= E, so the entry is in bounds even when the slot is idle)
      const int na = *src.n_active;
      const int e = src.active[slot];
      if (slot >= na) return false;
      bw.e = e;
      bw.p0 = src.offsets[e];
      bw.nrows = src.offsets[e + 1] - bw.p0;
    } else {
      bw.e = src.fixed_expert;
      bw.p0 = 0;
      bw.nrows = src.n_rows;
    }
  } else {
    bw.shared = true;
    const int tg = (int)(before % a.ntg_s);
    bw.rb_index = (int)(before / a.ntg_s);
    bw.e = 0;
    bw.p0 = tg * a.tok_s;
    bw.nrows = min(a.tok_s, a.n_tok - bw.p0);
  }
  return bw.nrows > 0;
}

__device__ __forceinline__ Job make_job(const GemvArgs& a, const BlockWork& bw, bool down) {
  Job jb;
  const ExpertSetDev& w = bw.shared ? a.ws : a.w;
  const MatGeo& g = bw.shared ? a.geo_s : a.geo;
  if (down) {
    jb.W = w.dn + (int64_t)bw.e * w.dn_stride;
    jb.S = reinterpret_cast<const float*>(w.dns + (int64_t)bw.e * w.dns_stride);
    jb.K = bw.shared ? a.Is : a.I;
    jb.rows = a.H;
  } else {
    jb.W = w.gu + (int64_t)bw.e * w.gu_stride;
    jb.S = reinterpret_cast<const float*>(w.gus + (int64_t)bw.e * w.gus_stride);
    jb.K = a.H;
    jb.rows = bw.shared ? a.Is : a.I;
  }
  jb.lpr = g.lpr;
  jb.rpp = g.rpp;
  const int rb = bw.shared ? a.rb_s : a.rb;
  jb.r0 = bw.rb_index * rb;
  jb.nr = rb;
  return jb;
}

// PRE: one routed gate/up row on the ring path whose activation slice and
// granule sums the caller has read already (xpre / gpre, as job_ring takes them).
// NATX: input rows in natural order are read by job_ring's NATX mode instead
// of being staged through the ring area.
template <int WDT, int KSL, int NTMAX, int ABF16, bool DOWN, bool PRE = false, bool NATX = false>
__device__ __forceinline__ void run_block(const GemvArgs& a, BlockWork bw, RingLds& L,
                                          const float* xpre = nullptr, const float* gpre = nullptr) {
  static_assert(!PRE || (NTMAX == 1 && !DOWN), "preloaded slices: one gate/up row at a time");
  const Job jb = make_job(a, bw, DOWN);
  if (jb.r0 >= jb.rows) return;
  const RowSource& src = a.src;
  const void* in = DOWN ? (bw.shared ? a.h_s : a.h) : (bw.shared && a.x_s ? a.x_s : a.x);
  void* out = DOWN ? (void*)(bw.shared ? a.y_s : a.y) : (bw.shared ? a.h_s : a.h);
  // 16-byte granules (and int8's 32-byte ones, as two slots, and int2's
  // 8-byte ones, two to a slot) on rows of >= 64 granules take the ring path
  // (the launcher keeps blocks within kMaxRingRows rows); slices longer than
  // one granule only occur on such rows, so the register path is compiled
  // for one-granule slices only
  constexpr bool kRingFmt = Fmt<WDT>::GB == 16 || WDT == MOE_I8 || WDT == MOE_I2;
  constexpr bool kChunk = !kRingFmt || KSL == Fmt<WDT>::EPG;
  constexpr int EPG = Fmt<WDT>::EPG, AB = ABF16 ? 2 : 4;
  const bool ring = kRingFmt && jb.lpr == 64;
  if (!ring && !kChunk) return;
  const int nr = min(jb.nr, jb.rows - jb.r0);
  static_assert(NTMAX == 1 || KSL <= 32, "two-token passes need short slices");
  constexpr int NT2 = NTMAX >= 2 ? 2 : 1;
  for (int i0 = 0; i0 < bw.nrows; i0 += NTMAX) {
    const int nt = min(NTMAX, bw.nrows - i0);
    int64_t xo[NTMAX], dr[NTMAX];
#pragma unroll
    for (int n = 0; n < NTMAX; ++n) {
      const int i = i0 + (n < nt ? n : 0);
      const int q = bw.p0 + i;   // bucket position, fixed-expert row or token
      // flat slot of a routed row
      const int f = (!bw.shared && src.routed) ? (bw.have_f ? (i == 0 ? bw.f0 : bw.f1) : src.entries[q]) : 0;
      if (DOWN) {
        xo[n] = (int64_t)q * jb.K;
        dr[n] = (!bw.shared && src.routed) ? (int64_t)f : (int64_t)q;
      } else {
        int t;
        if (bw.shared) t = q;
        else if (src.routed) t = f / src.top_k;
        else t = src.rows ? src.rows[q] / src.row_div : q;
        xo[n] = (int64_t)t * jb.K;
        dr[n] = q;
      }
    }
    if constexpr (kRingFmt) {
      if (ring) {
        if constexpr (PRE) {
          job_ring<WDT, KSL, 1, ABF16, !DOWN, true, true>(jb, nr, in, xo, 1, L, xpre, gpre);
        } else if (a.in_sliced) {
          if (NT2 == 2 && nt >= 2)
            job_ring<WDT, KSL, NT2, ABF16, !DOWN, true>(jb, nr, in, xo, nt, L);
          else
            job_ring<WDT, KSL, 1, ABF16, !DOWN, true>(jb, nr, in, xo, 1, L);
        } else if constexpr (NATX) {
          if (NT2 == 2 && nt >= 2)
            job_ring<WDT, KSL, NT2, ABF16, !DOWN, false, false, true>(jb, nr, in, xo, nt, L);
          else
            job_ring<WDT, KSL, 1, ABF16, !DOWN, false, false, true>(jb, nr, in, xo, 1, L);
        } else {
          if (NT2 == 2 && nt >= 2)
            job_ring<WDT, KSL, NT2, ABF16, !DOWN, false>(jb, nr, in, xo, nt, L);
          else
            job_ring<WDT, KSL, 1, ABF16, !DOWN, false>(jb, nr, in, xo, 1, L);
        }
        __syncthreads();
        const int ntw = (NT2 == 2 && nt >= 2) ? nt : 1;
        const bool sl = !DOWN && a.out_sliced;
        float* probe = DOWN ? nullptr : (bw.shared ? a.hp_s : a.hp);
        for (int t = threadIdx.x; t < ntw * nr; t += kThreads) {
          const int n = t / nr, rl = t - n * nr;
          const int64_t col = jb.r0 + rl;
          const int64_t o = dr[n] * jb.rows + (sl ? sliced_index(col, EPG, AB) : col);
          if (!DOWN && ABF16)
            reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16_bits(L.out[n][rl]);
          else
            reinterpret_cast<float*>(out)[o] = L.out[n][rl];
          if (probe) probe[dr[n] * jb.rows + col] = L.out[n][rl];
        }
        __syncthreads();
        continue;
      }
    }
    if constexpr (kChunk) {
      if (NT2 == 2 && nt >= 2)
        job_chunk<WDT, KSL, NT2, ABF16, !DOWN>(jb, in, xo, nt, out, dr,
                                               DOWN ? nullptr : (bw.shared ? a.hp_s : a.hp));
      else
        job_chunk<WDT, KSL, 1, ABF16, !DOWN>(jb, in, xo, 1, out, dr,
                                             DOWN ? nullptr : (bw.shared ? a.hp_s : a.hp));
    }
  }
}

// ------------------------------------------------------------------ kernels
// One launch covers the routed experts (n_slots x nb blocks; slots beyond
// n_active, or beyond the bucketed rows in token mode, exit at once) and,
// optionally, the shared expert (nb_s x ntg_s blocks).

template <int WR, int KR, int WS, int KS, int NTMAX, int ABF16, bool DOWN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_gemv(GemvArgs a) {
  __shared__ RingLds lds;
  BlockWork bw;
  if (!block_work(a, bw, blockIdx.x)) return;
  if (bw.shared)
    run_block<WS, KS, NTMAX, ABF16, DOWN>(a, bw, lds);
  else
    run_block<WR, KR, NTMAX, ABF16, DOWN>(a, bw, lds);
}

// A shared-expert launch whose first p.blocks blocks run routing work: the
// router logits of expert row blockIdx.x (gate/up launch) or, in one block,
// the selection and grouping (down launch).  Their LDS scratch is the ring
// area, so the launch keeps the GEMV's occupancy.
static_assert(sizeof(double) * kDecodeTokens * 256 <= sizeof(RingLds::ring), "logits scratch");
static_assert(sizeof(SelectBucketLds) <= sizeof(RingLds::ring), "selection scratch");

template <int WS, int KS, int ABF16, bool DOWN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8))) void k_gemv_pre(
    GemvArgs a, PreArgs p) {
  __shared__ RingLds lds;
  if ((int)blockIdx.x < p.blocks) {
    if constexpr (!DOWN) {
      logits_row_block(p.w_router, p.x, p.act_bf16, p.T, p.H, p.E, p.z, p.sr, blockIdx.x,
                       reinterpret_cast<double*>(&lds.ring[0][0][0]), p.zsc, p.zbias);
    } else {
      select_bucket_block<4, true>(p.sp, p.zin, p.bias, p.T, p.idx, p.w, p.counts, p.offsets,
                                   p.entries, p.inverse, p.active, p.n_active,
                                   *reinterpret_cast<SelectBucketLds*>(&lds.ring[0][0][0]), p.tb);
    }
    return;
  }
  BlockWork bw;
  if (!block_work(a, bw, (int64_t)blockIdx.x - p.blocks)) return;
  // the gate/up launch reads the layer input as it is: in natural order,
  // with the weight ring's first fill issued behind the activation loads
  run_block<WS, KS, 1, ABF16, DOWN, false, !DOWN>(a, bw, lds);
}

template <int WS, int KS, bool DOWN>
hipError_t gemv_pre_go(const GemvArgs& a, const PreArgs& p, int act_bf16, unsigned blocks,
                       hipStream_t s) {
  if (act_bf16)
    hipLaunchKernelGGL((k_gemv_pre<WS, KS, 1, DOWN>), dim3(blocks), dim3(kThreads), 0, s, a, p);
  else
    hipLaunchKernelGGL((k_gemv_pre<WS, KS, 0, DOWN>), dim3(blocks), dim3(kThreads), 0, s, a, p);
  return hipGetLastError();
}


template <int WR, int KR, int WS, int KS, bool DOWN>
hipError_t gemv_go(const GemvArgs& a, int ntmax, int act_bf16, unsigned blocks, hipStream_t s) {
#define MOE_K(NT, AB) \
  hipLaunchKernelGGL((k_gemv<WR, KR, WS, KS, NT, AB, DOWN>), dim3(blocks), dim3(kThreads), 0, s, a)
  if constexpr (KR <= 32 && WR != MOE_I8) {
    if (ntmax >= 2) {
      if (act_bf16) MOE_K(2, 1); else MOE_K(2, 0);
      return hipGetLastError();
    }
  }
  if (act_bf16) MOE_K(1, 1); else MOE_K(1, 0);
#undef MOE_K
  return hipGetLastError();
}

// Geometry, token mode and block sizes of a GEMV launch (k_gemv.hip); returns
// the number of blocks (0: no work) or -1 when a shape is not covered.
// ntmax: tokens one pass of a block takes; target_blocks: blocks of one
// resident round (2048 waves of 4-wave blocks).
long long plan_gemv(GemvArgs& a, bool down, int dtype, int& shared_dtype, int max_rows_per_slot,
                    bool allow_nt2, int& ntmax, int64_t target_blocks = 512);

// Per-format entry points (one translation unit each, compiled in parallel).
// The shared expert's slice length always equals the routed one (both K/64,
// or the same short-row geometry), so only its format varies.
hipError_t gemv_i4_gu(const GemvArgs&, int, int, int, unsigned, hipStream_t);
hipError_t gemv_i4_dn(const GemvArgs&, int, int, int, unsigned, hipStream_t);
hipError_t gemv_i2_gu(const GemvArgs&, int, int, int, unsigned, hipStream_t);
hipError_t gemv_i2_dn(const GemvArgs&, int, int, int, unsigned, hipStream_t);
hipError_t gemv_i8_gu(const GemvArgs&, int, int, int, unsigned, hipStream_t);
hipError_t gemv_i8_dn(const GemvArgs&, int, int, int, unsigned, hipStream_t);
hipError_t gemv_bf_gu(const GemvArgs&, int, int, int, unsigned, hipStream_t);
hipError_t gemv_bf_dn(const GemvArgs&, int, int, int, unsigned, hipStream_t);
// Shared-expert launches with leading routing blocks (shared format, K-slice
// length a.geo_s.kc).
hipError_t gemv_pre_gu(const GemvArgs&, const PreArgs&, int, int, unsigned, hipStream_t);
hipError_t gemv_pre_dn(const GemvArgs&, const PreArgs&, int, int, unsigned, hipStream_t);

}  // namespace moe
