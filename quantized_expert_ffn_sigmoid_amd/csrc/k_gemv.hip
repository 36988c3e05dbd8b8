// k_gemv.hip -- dequant-on-use expert GEMV for decode-sized buckets (gfx950).
//
// Experts are SwiGLU FFNs whose weights are packed int4 / packed int2 codes
// with one fp32 scale per output row, or bf16 ("colibri" README, "What's
// implemented": quantization kernels, per-row scales, dequant-on-use;
// "iliria" README, "What's implemented": routed-expert SwiGLU with gate and up
// over one activation).  Decode work is HBM-bound: every code byte is read
// once, so the kernel is organised around coalesced 16-byte loads and a
// minimal unpack, not around matrix cores.
//
// Layout of the work:
//  * a row of the [out][in] matrix is split into granules of 16 bytes (8 for
//    int2); lane j of a row group reads granules j, j+LPR, j+2LPR, ... so a
//    wave-wide load covers 64 consecutive granules (1 KB) of one row;
//  * each lane keeps the matching slice of the activation row(s) in
//    registers for the whole block, and the same lanes walk down the rows;
//  * codes are unpacked as offset-binary bytes (XOR of the sign bits, two
//    masks) and converted with the byte-to-float instructions; the offset is
//    removed once per row from the lane's activation-slice sum, and the per-row
//    scale is applied in the epilogue, since it is constant along the row;
//  * partial dot products are reduced across the row group with shuffles.
// Accumulation is fp32 throughout.
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

template <int WDT>
__device__ __forceinline__ void load_granule(const uint8_t* p, uint32_t (&g)[Fmt<WDT>::DW]) {
  if constexpr (Fmt<WDT>::DW == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    g[0] = v.x;
    g[1] = v.y;
    g[2] = v.z;
    g[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    g[0] = v.x;
    g[1] = v.y;
  }
}

// Granule -> EPG floats in K order.  int formats yield code + OFF.
template <int WDT>
__device__ __forceinline__ void unpack(const uint32_t (&g)[Fmt<WDT>::DW], float (&q)[Fmt<WDT>::EPG]) {
  if constexpr (WDT == MOE_I4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t w = g[d] ^ 0x88888888u;
      const uint32_t lo = w & 0x0F0F0F0Fu;
      const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        q[8 * d + 2 * b] = (float)((lo >> (8 * b)) & 0xFFu);
        q[8 * d + 2 * b + 1] = (float)((hi >> (8 * b)) & 0xFFu);
      }
    }
  } else if constexpr (WDT == MOE_I2) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint32_t w = g[d] ^ 0xAAAAAAAAu;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t c = (w >> (2 * jj)) & 0x03030303u;
#pragma unroll
        for (int b = 0; b < 4; ++b) q[16 * d + 4 * b + jj] = (float)((c >> (8 * b)) & 0xFFu);
      }
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      q[2 * d] = __uint_as_float(g[d] << 16);
      q[2 * d + 1] = __uint_as_float(g[d] & 0xFFFF0000u);
    }
  }
}

// Activation slice of one row: xs[g*EPG + c] = x[(g*LPR + j)*EPG + c].
template <int EPG, int GPL, int ABF16>
__device__ __forceinline__ void load_slice(const void* base, int64_t row_off, int LPR, int j,
                                           float (&xs)[GPL * EPG]) {
#pragma unroll
  for (int g = 0; g < GPL; ++g) {
    const int64_t k0 = row_off + (int64_t)(g * LPR + j) * EPG;
    if constexpr (ABF16) {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + k0;
#pragma unroll
      for (int c = 0; c < EPG; c += 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(p + c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          xs[g * EPG + c + 2 * d] = __uint_as_float(w[d] << 16);
          xs[g * EPG + c + 2 * d + 1] = __uint_as_float(w[d] & 0xFFFF0000u);
        }
      }
    } else {
      const float* p = reinterpret_cast<const float*>(base) + k0;
#pragma unroll
      for (int c = 0; c < EPG; c += 4) {
        const float4 v = *reinterpret_cast<const float4*>(p + c);
        xs[g * EPG + c] = v.x;
        xs[g * EPG + c + 1] = v.y;
        xs[g * EPG + c + 2] = v.z;
        xs[g * EPG + c + 3] = v.w;
      }
    }
  }
}

__device__ __forceinline__ float group_sum(float v, int LPR) {
  for (int m = LPR >> 1; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Resolve expert and row range of this block; false when the slot is idle.
__device__ __forceinline__ bool block_rows(const RowSource& src, int& e, int& p0, int& nrows) {
  if (src.routed) {
    const int slot = blockIdx.y;
    if (slot >= *src.n_active) return false;
    e = src.active[slot];
    p0 = src.offsets[e];
    nrows = src.offsets[e + 1] - p0;
  } else {
    e = src.fixed_expert;
    p0 = 0;
    nrows = src.n_rows;
  }
  return true;
}

__device__ __forceinline__ int token_of(const RowSource& src, int p0, int i) {
  if (src.routed) return src.entries[p0 + i] / src.top_k;
  return src.rows ? src.rows[i] / src.row_div : i;
}

constexpr int kPasses = 4;   // row passes per wave
constexpr int kBlockWaves = 4;

// ------------------------------------------------------------- gate / up
template <int WDT, int KSL, int NT, int ABF16>
__global__ __launch_bounds__(256) void k_gemv_gate_up(GemvGateUpArgs a) {
  using F = Fmt<WDT>;
  constexpr int EPG = F::EPG, GB = F::GB, DW = F::DW, GPL = KSL / EPG;
  int e, p0, nrows;
  if (!block_rows(a.src, e, p0, nrows)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.H, I = a.I;
  const int LPR = H / KSL, RPP = kWave / LPR;
  const int j = lane & (LPR - 1), rg = lane / LPR;
  const int64_t rbytes = (int64_t)(H / EPG) * GB;
  const uint8_t* W = a.w.gu + (int64_t)e * a.w.gu_stride;
  const float* S = nullptr;
  if constexpr (WDT != MOE_BF16) S = reinterpret_cast<const float*>(a.w.gus + (int64_t)e * a.w.gus_stride);
  const int rbase = (blockIdx.x * kBlockWaves + wave) * kPasses * RPP;
  if (rbase >= I) return;

  for (int i0 = blockIdx.z * NT; i0 < nrows; i0 += gridDim.z * NT) {
    float xs[NT][KSL];
    float xsum[NT];
    int hrow[NT];
    bool tv[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int i = i0 + n;
      tv[n] = i < nrows;
      const int t = token_of(a.src, p0, tv[n] ? i : i0);
      hrow[n] = p0 + i;
      load_slice<EPG, GPL, ABF16>(a.x, (int64_t)t * H, LPR, j, xs[n]);
      float sx = 0.f;
#pragma unroll
      for (int c = 0; c < KSL; ++c) sx += xs[n][c];
      xsum[n] = sx;
    }
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const int r = rbase + ps * RPP + rg;
      const bool rv = r < I;
      const int rr = rv ? r : I - 1;
      const uint8_t* gp = W + (int64_t)rr * rbytes;
      const uint8_t* up = W + (int64_t)(I + rr) * rbytes;
      uint32_t cg[GPL][DW], cu[GPL][DW];
#pragma unroll
      for (int g = 0; g < GPL; ++g) {
        const int64_t off = (int64_t)(g * LPR + j) * GB;
        load_granule<WDT>(gp + off, cg[g]);
        load_granule<WDT>(up + off, cu[g]);
      }
      float ag[NT], au[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) ag[n] = au[n] = 0.f;
#pragma unroll
      for (int g = 0; g < GPL; ++g) {
        float qg[EPG], qu[EPG];
        unpack<WDT>(cg[g], qg);
        unpack<WDT>(cu[g], qu);
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int c = 0; c < EPG; ++c) {
            ag[n] = fmaf(qg[c], xs[n][g * EPG + c], ag[n]);
            au[n] = fmaf(qu[c], xs[n][g * EPG + c], au[n]);
          }
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if constexpr (WDT != MOE_BF16) {
          ag[n] = fmaf(-F::OFF, xsum[n], ag[n]);
          au[n] = fmaf(-F::OFF, xsum[n], au[n]);
        }
        ag[n] = group_sum(ag[n], LPR);
        au[n] = group_sum(au[n], LPR);
      }
      if (rv) {
        float sg = 1.f, su = 1.f;
        if constexpr (WDT != MOE_BF16) {
          sg = S[rr];
          su = S[I + rr];
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          if (j == (n & (LPR - 1)) && tv[n]) {
            const float gv = ag[n] * sg, uv = au[n] * su;
            const float hv = gv / (1.0f + expf(-gv)) * uv;
            if constexpr (ABF16)
              reinterpret_cast<uint16_t*>(a.h)[(int64_t)hrow[n] * I + r] = f32_to_bf16_bits(hv);
            else
              reinterpret_cast<float*>(a.h)[(int64_t)hrow[n] * I + r] = hv;
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------- down
template <int WDT, int KSL, int NT, int ABF16>
__global__ __launch_bounds__(256) void k_gemv_down(GemvDownArgs a) {
  using F = Fmt<WDT>;
  constexpr int EPG = F::EPG, GB = F::GB, DW = F::DW, GPL = KSL / EPG;
  int e, p0, nrows;
  if (!block_rows(a.src, e, p0, nrows)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.H, I = a.I;
  const int LPR = I / KSL, RPP = kWave / LPR;
  const int j = lane & (LPR - 1), rg = lane / LPR;
  const int64_t rbytes = (int64_t)(I / EPG) * GB;
  const uint8_t* W = a.w.dn + (int64_t)e * a.w.dn_stride;
  const float* S = nullptr;
  if constexpr (WDT != MOE_BF16) S = reinterpret_cast<const float*>(a.w.dns + (int64_t)e * a.w.dns_stride);
  const int obase = (blockIdx.x * kBlockWaves + wave) * kPasses * RPP;
  if (obase >= H) return;

  for (int i0 = blockIdx.z * NT; i0 < nrows; i0 += gridDim.z * NT) {
    float xs[NT][KSL];
    float xsum[NT];
    int64_t yrow[NT];
    bool tv[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int i = i0 + n;
      tv[n] = i < nrows;
      const int ii = tv[n] ? i : i0;
      const int64_t hr = p0 + ii;
      yrow[n] = a.src.routed ? (int64_t)a.src.entries[p0 + ii] : (int64_t)ii;
      load_slice<EPG, GPL, ABF16>(a.h, hr * I, LPR, j, xs[n]);
      float sx = 0.f;
#pragma unroll
      for (int c = 0; c < KSL; ++c) sx += xs[n][c];
      xsum[n] = sx;
    }
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const int o = obase + ps * RPP + rg;
      const bool ov = o < H;
      const int oo = ov ? o : H - 1;
      const uint8_t* wp = W + (int64_t)oo * rbytes;
      uint32_t cw[GPL][DW];
#pragma unroll
      for (int g = 0; g < GPL; ++g) load_granule<WDT>(wp + (int64_t)(g * LPR + j) * GB, cw[g]);
      float acc[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] = 0.f;
#pragma unroll
      for (int g = 0; g < GPL; ++g) {
        float q[EPG];
        unpack<WDT>(cw[g], q);
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int c = 0; c < EPG; ++c) acc[n] = fmaf(q[c], xs[n][g * EPG + c], acc[n]);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if constexpr (WDT != MOE_BF16) acc[n] = fmaf(-F::OFF, xsum[n], acc[n]);
        acc[n] = group_sum(acc[n], LPR);
      }
      if (ov) {
        float sc = 1.f;
        if constexpr (WDT != MOE_BF16) sc = S[oo];
#pragma unroll
        for (int n = 0; n < NT; ++n)
          if (j == (n & (LPR - 1)) && tv[n]) a.y[yrow[n] * H + o] = acc[n] * sc;
      }
    }
  }
}

// --------------------------------------------------------------- dispatch

template <int WDT>
static int pick_ksl(int32_t K) {
  // smallest instantiated K-slice with K / KSL a power of two <= 64
  const int cand_bf16[] = {8, 16, 32, 64, 96};
  const int cand_int[] = {32, 64, 96};
  const int* c = WDT == MOE_BF16 ? cand_bf16 : cand_int;
  const int n = WDT == MOE_BF16 ? 5 : 3;
  for (int i = 0; i < n; ++i) {
    if (K % c[i]) continue;
    const int lpr = K / c[i];
    if (lpr <= 64 && (lpr & (lpr - 1)) == 0) return c[i];
  }
  return 0;
}

bool gemv_supported(int dtype, int32_t K) {
  if (K <= 0) return false;
  if (dtype == MOE_I4) return pick_ksl<MOE_I4>(K) != 0;
  if (dtype == MOE_I2) return pick_ksl<MOE_I2>(K) != 0;
  if (dtype == MOE_BF16) return pick_ksl<MOE_BF16>(K) != 0;
  return false;
}

static dim3 gemv_grid(int rows, int K, int ksl, int slots, int max_rows, int nt) {
  const int lpr = K / ksl, rpp = kWave / lpr;
  const int rows_per_block = kBlockWaves * kPasses * rpp;
  const int gx = (rows + rows_per_block - 1) / rows_per_block;
  int gz = (max_rows + nt - 1) / nt;
  if (gz < 1) gz = 1;
  if (gz > 32) gz = 32;
  return dim3(gx, slots, gz);
}

template <int WDT, int KSL, int NT>
static hipError_t launch_gu3(const GemvGateUpArgs& a, int act_bf16, dim3 grid, hipStream_t s) {
  if (act_bf16)
    hipLaunchKernelGGL((k_gemv_gate_up<WDT, KSL, NT, 1>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemv_gate_up<WDT, KSL, NT, 0>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int WDT, int KSL, int NT>
static hipError_t launch_dn3(const GemvDownArgs& a, int act_bf16, dim3 grid, hipStream_t s) {
  if (act_bf16)
    hipLaunchKernelGGL((k_gemv_down<WDT, KSL, NT, 1>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemv_down<WDT, KSL, NT, 0>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int WDT, int KSL>
static hipError_t launch_gu2(const GemvGateUpArgs& a, int act_bf16, int nt, dim3 grid, hipStream_t s) {
  if (nt == 1) return launch_gu3<WDT, KSL, 1>(a, act_bf16, grid, s);
  return launch_gu3<WDT, KSL, 2>(a, act_bf16, grid, s);
}

template <int WDT, int KSL>
static hipError_t launch_dn2(const GemvDownArgs& a, int act_bf16, int nt, dim3 grid, hipStream_t s) {
  if (nt == 1) return launch_dn3<WDT, KSL, 1>(a, act_bf16, grid, s);
  return launch_dn3<WDT, KSL, 2>(a, act_bf16, grid, s);
}

template <int WDT>
static hipError_t launch_gu1(const GemvGateUpArgs& a, int act_bf16, int slots, int max_rows,
                             hipStream_t s) {
  const int ksl = pick_ksl<WDT>(a.H);
  const int nt = max_rows <= 1 ? 1 : 2;
  const dim3 grid = gemv_grid(a.I, a.H, ksl, slots, max_rows, nt);
  switch (ksl) {
    case 32: return launch_gu2<WDT, 32>(a, act_bf16, nt, grid, s);
    case 64: return launch_gu2<WDT, 64>(a, act_bf16, nt, grid, s);
    case 96: return launch_gu2<WDT, 96>(a, act_bf16, nt, grid, s);
    default: break;
  }
  if constexpr (WDT == MOE_BF16) {
    if (ksl == 8) return launch_gu2<WDT, 8>(a, act_bf16, nt, grid, s);
    if (ksl == 16) return launch_gu2<WDT, 16>(a, act_bf16, nt, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int WDT>
static hipError_t launch_dn1(const GemvDownArgs& a, int act_bf16, int slots, int max_rows,
                             hipStream_t s) {
  const int ksl = pick_ksl<WDT>(a.I);
  const int nt = max_rows <= 1 ? 1 : 2;
  const dim3 grid = gemv_grid(a.H, a.I, ksl, slots, max_rows, nt);
  switch (ksl) {
    case 32: return launch_dn2<WDT, 32>(a, act_bf16, nt, grid, s);
    case 64: return launch_dn2<WDT, 64>(a, act_bf16, nt, grid, s);
    case 96: return launch_dn2<WDT, 96>(a, act_bf16, nt, grid, s);
    default: break;
  }
  if constexpr (WDT == MOE_BF16) {
    if (ksl == 8) return launch_dn2<WDT, 8>(a, act_bf16, nt, grid, s);
    if (ksl == 16) return launch_dn2<WDT, 16>(a, act_bf16, nt, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_gate_up(const GemvGateUpArgs& a, int dtype, int act_bf16, int max_slots,
                               int max_rows_per_slot, hipStream_t s) {
  if (max_slots <= 0 || max_rows_per_slot <= 0) return hipSuccess;
  switch (dtype) {
    case MOE_I4: return launch_gu1<MOE_I4>(a, act_bf16, max_slots, max_rows_per_slot, s);
    case MOE_I2: return launch_gu1<MOE_I2>(a, act_bf16, max_slots, max_rows_per_slot, s);
    case MOE_BF16: return launch_gu1<MOE_BF16>(a, act_bf16, max_slots, max_rows_per_slot, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv_down(const GemvDownArgs& a, int dtype, int act_bf16, int max_slots,
                            int max_rows_per_slot, hipStream_t s) {
  if (max_slots <= 0 || max_rows_per_slot <= 0) return hipSuccess;
  switch (dtype) {
    case MOE_I4: return launch_dn1<MOE_I4>(a, act_bf16, max_slots, max_rows_per_slot, s);
    case MOE_I2: return launch_dn1<MOE_I2>(a, act_bf16, max_slots, max_rows_per_slot, s);
    case MOE_BF16: return launch_dn1<MOE_BF16>(a, act_bf16, max_slots, max_rows_per_slot, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
