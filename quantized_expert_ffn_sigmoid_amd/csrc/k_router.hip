// k_router.hip -- RMSNorm, router logits (fp64) and expert selection for gfx950.
//
// Router ("colibri" README, "What's implemented": DeepSeek-V3-style sigmoid
// router, noaux_tc, routed_scaling_factor; Granite MoE softmax top-k router on
// the "Glacial" page).  Logits accumulate exact fp32 products in fp64 so that
// the selected indices are reproducible against an fp64 reference: two
// orderings of an fp64 sum differ by ~1e-16 relative, far below the gaps
// between distinct scores of continuous data.
#include "route_device.h"

namespace moe {

// ------------------------------------------------------------------ RMSNorm
// One block per token.  Sum of squares in fp64 (each square of a float is exact
// in fp64), then out = float(x / sqrt(mean + eps)) with an IEEE fp64 divide.
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ x,
                                                 float* __restrict__ out, int32_t H, float eps) {
  __shared__ double red[256];
  const int64_t t = blockIdx.x;
  const float* xr = x + t * H;
  double ss = 0.0;
  for (int h = threadIdx.x; h < H; h += 256) {
    double v = (double)xr[h];
    ss += v * v;
  }
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double den = sqrt(red[0] / (double)H + (double)eps);
  for (int h = threadIdx.x; h < H; h += 256) out[t * H + h] = (float)((double)xr[h] / den);
}

hipError_t launch_rmsnorm(const float* x, float* out, int32_t T, int32_t H, float eps,
                          hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm, dim3(T), dim3(256), 0, s, x, out, H, eps);
  return hipGetLastError();
}

// ----------------------------------------------------------- router logits

// Decode shape (T <= 16): one block of 256 threads per expert row
// (logits_row_block).
__global__ __launch_bounds__(256) void k_logits_gemv(const float* __restrict__ W,
                                                     const void* __restrict__ x, int act_bf16,
                                                     int32_t T, int32_t H, int32_t E,
                                                     double* __restrict__ z, SliceReq sr) {
  __shared__ double red[kDecodeTokens][256];
  logits_row_block(W, x, act_bf16, T, H, E, z, sr, blockIdx.x, &red[0][0]);
}

// Prefill shape: 64 tokens x 64 experts per block on the fp64 matrix cores
// (v_mfma_f64_16x16x4_f64): the fp32 operands are widened to fp64 when staged
// in LDS, so every product is exact and each output is summed in fp64, four
// K values per instruction in K order.  Each of the 4 waves owns a 32 x 32
// quadrant (2 x 2 instruction tiles).  Operand layout of the instruction:
// lane l supplies A[l % 16][l / 16] (token row, K) and B[l / 16][l % 16]
// (K, expert column) and receives D[l / 16 + 4 r][l % 16], r = 0..3.
// With split K (gridDim.z chunks of kc), chunk c writes its partial sums to
// z + c * T * E and k_logits_reduce adds the chunks in order.
constexpr int LG_BT = 64, LG_BE = 64, LG_BK = 16;
__global__ __launch_bounds__(256) void k_logits_gemm(const float* __restrict__ W,
                                                     const void* __restrict__ x, int act_bf16,
                                                     int32_t T, int32_t H, int32_t E, int32_t kc,
                                                     double* __restrict__ z) {
  // operands widened to fp64 once, when staged (each is read by the two
  // waves whose quadrants share its rows or columns)
  __shared__ double sx[LG_BK][LG_BT + 2];
  __shared__ double sw[LG_BK][LG_BE + 2];
  const int t0 = blockIdx.x * LG_BT, e0 = blockIdx.y * LG_BE;
  const int kbeg = blockIdx.z * kc, kend = kbeg + kc;
  z += (int64_t)blockIdx.z * T * E;
  typedef double f64x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qr = (wave >> 1) * 32, qc = (wave & 1) * 32;   // the wave's quadrant
  const int li = lane & 15, lk = lane >> 4;
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  // each thread stages 4 consecutive k of one row of x and of W; the next
  // step's values are loaded into registers while the current step computes
  const int lr = threadIdx.x >> 2, sk = (threadIdx.x & 3) * 4;
  const int t = t0 + lr, e = e0 + lr;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f), w = make_float4(0.f, 0.f, 0.f, 0.f);
  auto load = [&](int k0) {
    if (t < T) v = load_x4(x, act_bf16, (int64_t)t * H + k0 + sk);
    if (e < E) w = *reinterpret_cast<const float4*>(W + (int64_t)e * H + k0 + sk);
  };
  // workgroup barrier after this wave's LDS accesses, without the release
  // fence of __syncthreads (which would also wait for the loads in flight)
  auto lds_barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  if (kbeg < kend) load(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += LG_BK) {
    sx[sk + 0][lr] = (double)v.x;
    sx[sk + 1][lr] = (double)v.y;
    sx[sk + 2][lr] = (double)v.z;
    sx[sk + 3][lr] = (double)v.w;
    sw[sk + 0][lr] = (double)w.x;
    sw[sk + 1][lr] = (double)w.y;
    sw[sk + 2][lr] = (double)w.z;
    sw[sk + 3][lr] = (double)w.w;
    lds_barrier();
    if (k0 + LG_BK < kend) load(k0 + LG_BK);
#pragma unroll
    for (int k = 0; k < LG_BK; k += 4) {
      double a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = sx[k + lk][qr + 16 * i + li];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = sw[k + lk][qc + 16 * j + li];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    lds_barrier();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + qr + 16 * i + lk + 4 * r;
      if (t >= T) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = e0 + qc + 16 * j + li;
        if (e < E) z[(int64_t)t * E + e] = acc[i][j][r];
      }
    }
  }
}

// Chunked sums added in chunk order: z = ((p0 + p1) + p2) + ...
__global__ __launch_bounds__(256) void k_logits_reduce(const double* __restrict__ part, int32_t n_chunks,
                                                       int64_t n, double* __restrict__ z) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    double v = part[i];
    for (int c = 1; c < n_chunks; ++c) v += part[(int64_t)c * n + i];
    z[i] = v;
  }
}

hipError_t launch_router_logits(const float* w_router, const void* x, int act_bf16, int32_t T,
                                int32_t H, int32_t E, double* z, const SliceReq& sr,
                                hipStream_t s, double* zpart, int64_t zpart_elems) {
  if (T <= 0) return hipSuccess;
  if (T <= kDecodeTokens) {
    hipLaunchKernelGGL(k_logits_gemv, dim3(E), dim3(256), 0, s, w_router, x, act_bf16, T, H, E,
                       z, sr);
  } else {
    if (sr.dst_a || sr.dst_b) {
      const hipError_t st = launch_slice_rows(x, act_bf16, T, H, sr.epg_a, sr.dst_a, sr.epg_b,
                                              sr.dst_b, s);
      if (st != hipSuccess) return st;
    }
    // split K so that the grid fills the chip (about 1024 blocks), when a
    // scratch area for the partial sums is given; H is a multiple of 32
    const int64_t tiles = (int64_t)((T + LG_BT - 1) / LG_BT) * ((E + LG_BE - 1) / LG_BE);
    int chunks = 1;
    if (zpart) {
      int want = (int)((1024 + tiles - 1) / tiles);
      if (want > 8) want = 8;
      for (int c = want; c > 1; --c)
        if ((H / LG_BK) % c == 0 && (int64_t)c * T * E <= zpart_elems) {
          chunks = c;
          break;
        }
    }
    dim3 grid((T + LG_BT - 1) / LG_BT, (E + LG_BE - 1) / LG_BE, chunks);
    hipLaunchKernelGGL(k_logits_gemm, grid, dim3(256), 0, s, w_router, x, act_bf16, T, H, E,
                       H / chunks, chunks > 1 ? zpart : z);
    if (chunks > 1) {
      const int64_t n = (int64_t)T * E;
      int64_t blocks = (n + 255) / 256;
      if (blocks > 4096) blocks = 4096;
      hipLaunchKernelGGL(k_logits_reduce, dim3((unsigned)blocks), dim3(256), 0, s, zpart, chunks,
                         n, z);
    }
  }
  return hipGetLastError();
}

template <int EPL>
__global__ __launch_bounds__(256) void k_select(SelectParams p, const double* __restrict__ z,
                                                const float* __restrict__ bias, int32_t T,
                                                int32_t* __restrict__ topk_idx,
                                                float* __restrict__ topk_w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (p.softmax)
    select_token<EPL, true>(p, z + (int64_t)t * p.E, bias, topk_idx + (int64_t)t * p.K,
                            topk_w + (int64_t)t * p.K, nullptr);
  else
    select_token<EPL, false>(p, z + (int64_t)t * p.E, bias, topk_idx + (int64_t)t * p.K,
                             topk_w + (int64_t)t * p.K, nullptr);
}

// Decode: selection of all T <= 16 tokens (one wave each) and the grouping,
// in one block (select_bucket_block).
template <int EPL>
__global__ __launch_bounds__(256) void k_select_bucket(
    SelectParams p, const double* __restrict__ z, const float* __restrict__ bias, int32_t T,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ entries, int32_t* __restrict__ inverse,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, SlotTables tb) {
  __shared__ SelectBucketLds L;
  select_bucket_block<EPL>(p, z, bias, T, topk_idx, topk_w, counts, offsets, entries, inverse,
                           active, n_active, L, tb);
}

SelectParams select_params(const moe_layer_desc& d) {
  SelectParams p;
  p.E = d.n_experts;
  p.K = d.top_k;
  p.softmax = d.router == MOE_ROUTER_SOFTMAX_TOPK;
  p.G = p.softmax ? 1 : d.n_group;
  p.topk_group = p.softmax ? 1 : d.topk_group;
  p.scaling = d.routed_scaling;
  p.top_p = (double)d.top_p;
  p.zsc = nullptr;
  return p;
}

hipError_t launch_router_select(const moe_layer_desc& d, const double* z, const float* bias,
                                int32_t T, int32_t* topk_idx, float* topk_w, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const SelectParams p = select_params(d);
  const dim3 grid((T + 3) / 4), block(256);
  const int epl = (d.n_experts + 63) / 64;
#define MOE_SEL(N) hipLaunchKernelGGL(k_select<N>, grid, block, 0, s, p, z, bias, T, topk_idx, topk_w)
  if (epl <= 1) MOE_SEL(1);
  else if (epl <= 2) MOE_SEL(2);
  else if (epl <= 4) MOE_SEL(4);
  else if (epl <= 8) MOE_SEL(8);
  else MOE_SEL(16);
#undef MOE_SEL
  return hipGetLastError();
}

hipError_t launch_select_bucket(const moe_layer_desc& d, const double* z, const float* bias,
                                int32_t T, int32_t* topk_idx, float* topk_w, int32_t* counts,
                                int32_t* offsets, int32_t* entries, int32_t* inverse,
                                int32_t* active, int32_t* n_active, hipStream_t s,
                                const SlotTables& tb) {
  if (T <= 0 || T > kDecodeTokens) return hipErrorInvalidValue;
  const SelectParams p = select_params(d);
  const int epl = (d.n_experts + 63) / 64;
#define MOE_SB(N)                                                                            \
  hipLaunchKernelGGL(k_select_bucket<N>, dim3(1), dim3(256), 0, s, p, z, bias, T,            \
                     topk_idx, topk_w, counts, offsets, entries, inverse, active, n_active, tb)
  if (epl <= 1) MOE_SB(1);
  else if (epl <= 2) MOE_SB(2);
  else if (epl <= 4) MOE_SB(4);
  else if (epl <= 8) MOE_SB(8);
  else MOE_SB(16);
#undef MOE_SB
  return hipGetLastError();
}

}  // namespace moe
