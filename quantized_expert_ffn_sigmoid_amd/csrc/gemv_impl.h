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
// int2).  A "unit" is one K-chunk of 64 granules of one row (of a gate/up row
// pair for the gate/up kernel): the 64 lanes of a wave load it as one 1 KB
// contiguous read.  Rows shorter than 64 granules put several rows in one
// unit (lanes-per-row LPR < 64).  A block owns a range of rows of one matrix
// and deals its units round-robin to its waves; each wave issues the loads of
// its next unit before computing the current one.  Activation rows are staged
// once per block in LDS in a lane-major layout (each ds_read_b128 of a wave
// touches 64 consecutive 16-byte slots, no bank conflicts).  Per-unit partial
// sums are reduced across the unit's lanes with shuffles and across K-chunks
// in LDS; the epilogue applies the per-row scale (constant along a row, so it
// commutes with the K-sum), SwiGLU, and writes h or y.
//
// Codes are unpacked as offset-binary bytes: XOR of the sign bits, two masks,
// then the byte-to-float conversions; the offset times the lane's activation
// sum is removed once per unit.  Accumulation is fp32 throughout.
#pragma once

#include "moe_internal.h"

namespace moe {

template <int WDT>
struct Fmt;
template <>
struct Fmt<MOE_I4> {
  static constexpr int EPG = 32, GB = 16, DW = 4;
  static constexpr float OFF = 8.0f;
};
template <>
struct Fmt<MOE_I2> {
  static constexpr int EPG = 32, GB = 8, DW = 2;
  static constexpr float OFF = 2.0f;
};
template <>
struct Fmt<MOE_BF16> {
  static constexpr int EPG = 8, GB = 16, DW = 4;
  static constexpr float OFF = 0.0f;
};

// Keeps the optimiser from folding the byte masks into 4-bit field extracts,
// so that each code converts with one v_cvt_f32_ubyteN.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Codes are streamed once: non-temporal loads keep them from displacing the
// activations and router weights in the caches.
template <int WDT>
__device__ __forceinline__ void load_granule(const uint8_t* p, uint32_t (&g)[Fmt<WDT>::DW]) {
  if constexpr (Fmt<WDT>::DW == 4) {
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
      const uint32_t w = gr[d] ^ 0x88888888u;
      const uint32_t lo = opaque(w & 0x0F0F0F0Fu);
      const uint32_t hi = opaque((w >> 4) & 0x0F0F0F0Fu);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float ql = (float)((lo >> (8 * b)) & 0xFFu);
        const float qh = (float)((hi >> (8 * b)) & 0xFFu);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          acc[n] = fmaf(ql, x[n][b0 + 8 * d + 2 * b], acc[n]);
          acc[n] = fmaf(qh, x[n][b0 + 8 * d + 2 * b + 1], acc[n]);
        }
      }
    }
  } else if constexpr (WDT == MOE_I2) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint32_t w = gr[d] ^ 0xAAAAAAAAu;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t c = opaque((w >> (2 * jj)) & 0x03030303u);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float q = (float)((c >> (8 * b)) & 0xFFu);
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[n] = fmaf(q, x[n][b0 + 16 * d + 4 * b + jj], acc[n]);
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

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL,
                                                    0xF, 0xF, false));
}

// Sum over aligned groups of lpr lanes (a power of two); every lane of a group
// receives the group's sum.  The first four steps are DPP register moves
// (quad swaps, then the 8- and 16-lane mirrors), the last two LDS permutes.
__device__ __forceinline__ float group_sum(float v, int lpr) {
  if (lpr >= 2) v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  if (lpr >= 4) v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  if (lpr >= 8) v += dpp_f<0x141>(v);   // row_half_mirror
  if (lpr >= 16) v += dpp_f<0x140>(v);  // row_mirror
  if (lpr >= 32) v += __shfl_xor(v, 16, kWave);
  if (lpr >= 64) v += __shfl_xor(v, 32, kWave);
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
// granules take GPL / CG steps).  CG * NM <= 6 keeps a step at <= 96 bytes
// per lane; PF steps are in flight while one is computed.
template <int GPL, int NM>
struct StepShape {
  static constexpr int cg_for(int c) { return (GPL % c == 0 && c * NM <= 6) ? c : cg_for(c - 1); }
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
                          void* dst, const int64_t* drow) {
  using F = Fmt<WDT>;
  constexpr int EPG = F::EPG, GB = F::GB, DW = F::DW, GPL = KSL / EPG;
  constexpr int NM = PAIR ? 2 : 1;
  using SS = StepShape<GPL, NM>;
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
                    acc[m][n] = fmaf(-F::OFF, gs[n][s2 * CG + g], acc[m][n]);
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
              sa = scale[0];
              if constexpr (PAIR) sb = scale[NM - 1];
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

// Which matrix and which token rows a block handles.
struct BlockWork {
  bool shared;
  int e, p0, nrows, rb_index;
};

__device__ __forceinline__ bool block_work(const GemvArgs& a, BlockWork& bw) {
  const int bid = blockIdx.x;
  const int routed_blocks = a.n_slots * a.nb;
  if (bid < routed_blocks) {
    const int slot = bid / a.nb;
    bw.shared = false;
    bw.rb_index = bid - slot * a.nb;
    const RowSource& src = a.src;
    if (src.routed) {
      if (slot >= *src.n_active) return false;
      bw.e = src.active[slot];
      bw.p0 = src.offsets[bw.e];
      bw.nrows = src.offsets[bw.e + 1] - bw.p0;
    } else {
      bw.e = src.fixed_expert;
      bw.p0 = 0;
      bw.nrows = src.n_rows;
    }
  } else {
    bw.shared = true;
    bw.rb_index = bid - routed_blocks;
    bw.e = 0;
    bw.p0 = 0;
    bw.nrows = a.n_tok;
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

template <int WDT, int KSL, int NTMAX, int ABF16, bool DOWN>
__device__ void run_block(const GemvArgs& a, const BlockWork& bw) {
  const Job jb = make_job(a, bw, DOWN);
  if (jb.r0 >= jb.rows) return;
  const RowSource& src = a.src;
  const void* in = DOWN ? (bw.shared ? a.h_s : a.h) : a.x;
  void* out = DOWN ? (void*)(bw.shared ? a.y_s : a.y) : (bw.shared ? a.h_s : a.h);
  for (int i0 = 0; i0 < bw.nrows; i0 += NTMAX) {
    const int nt = min(NTMAX, bw.nrows - i0);
    int64_t xo[NTMAX], dr[NTMAX];
#pragma unroll
    for (int n = 0; n < NTMAX; ++n) {
      const int i = i0 + (n < nt ? n : 0);
      if (DOWN) {
        xo[n] = ((int64_t)bw.p0 + i) * jb.K;
        dr[n] = (!bw.shared && src.routed) ? (int64_t)src.entries[bw.p0 + i] : (int64_t)i;
      } else {
        int t;
        if (bw.shared) t = i;
        else if (src.routed) t = src.entries[bw.p0 + i] / src.top_k;
        else t = src.rows ? src.rows[i] / src.row_div : i;
        xo[n] = (int64_t)t * jb.K;
        dr[n] = (int64_t)bw.p0 + i;
      }
    }
    if (NTMAX >= 2 && KSL <= 64 && nt >= 2)
      job_chunk<WDT, KSL, (NTMAX >= 2 && KSL <= 64 ? 2 : 1), ABF16, !DOWN>(jb, in, xo, nt, out, dr);
    else
      job_chunk<WDT, KSL, 1, ABF16, !DOWN>(jb, in, xo, 1, out, dr);
  }
}

// ------------------------------------------------------------------ kernels
// One launch covers the routed experts (n_slots x nb blocks; slots beyond
// n_active exit at once) and, optionally, the shared expert (nb_s blocks).

template <int WR, int KR, int WS, int KS, int NTMAX, int ABF16, bool DOWN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(KR > 64 || KS > 64 ? 2 : 3, 8))) void k_gemv(GemvArgs a) {
  BlockWork bw;
  if (!block_work(a, bw)) return;
  if (bw.shared)
    run_block<WS, KS, NTMAX, ABF16, DOWN>(a, bw);
  else
    run_block<WR, KR, NTMAX, ABF16, DOWN>(a, bw);
}


template <int WR, int KR, int WS, int KS, bool DOWN>
hipError_t gemv_go(const GemvArgs& a, int ntmax, int act_bf16, unsigned blocks, hipStream_t s) {
#define MOE_K(NT, AB) \
  hipLaunchKernelGGL((k_gemv<WR, KR, WS, KS, NT, AB, DOWN>), dim3(blocks), dim3(kThreads), 0, s, a)
  if constexpr (KR <= 64) {
    if (ntmax >= 2) {
      if (act_bf16) MOE_K(2, 1); else MOE_K(2, 0);
      return hipGetLastError();
    }
  }
  if (act_bf16) MOE_K(1, 1); else MOE_K(1, 0);
#undef MOE_K
  return hipGetLastError();
}

// Per-format entry points (one translation unit each, compiled in parallel).
// The shared expert's slice length always equals the routed one (both K/64,
// or the same short-row geometry), so only its format varies.
hipError_t gemv_i4_gu(const GemvArgs&, int, int, int, unsigned, hipStream_t);
hipError_t gemv_i4_dn(const GemvArgs&, int, int, int, unsigned, hipStream_t);
hipError_t gemv_i2_gu(const GemvArgs&, int, int, int, unsigned, hipStream_t);
hipError_t gemv_i2_dn(const GemvArgs&, int, int, int, unsigned, hipStream_t);
hipError_t gemv_bf_gu(const GemvArgs&, int, int, int, unsigned, hipStream_t);
hipError_t gemv_bf_dn(const GemvArgs&, int, int, int, unsigned, hipStream_t);

}  // namespace moe
