// k_router.hip -- RMSNorm, router logits (fp64) and expert selection for gfx950.
//
// Router ("colibri" README, "What's implemented": DeepSeek-V3-style sigmoid
// router, noaux_tc, routed_scaling_factor; Granite MoE softmax top-k router on
// the "Glacial" page).  Logits accumulate exact fp32 products in fp64 so that
// the selected indices are reproducible against an fp64 reference: two
// orderings of an fp64 sum differ by ~1e-16 relative, far below the gaps
// between distinct scores of continuous data.
#include "moe_internal.h"

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

__device__ __forceinline__ float4 load_x4(const void* x, int act_bf16, int64_t off) {
  if (act_bf16) {
    uint2 b = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + off);
    return make_float4(bf16_bits_to_f32(b.x & 0xFFFFu), bf16_bits_to_f32(b.x >> 16),
                       bf16_bits_to_f32(b.y & 0xFFFFu), bf16_bits_to_f32(b.y >> 16));
  }
  return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
}

// Decode shape (T <= 16): one wave per expert row; the row of W_r streams
// through with 16-byte loads, tokens are re-read from L1/L2.
__global__ __launch_bounds__(256) void k_logits_gemv(const float* __restrict__ W,
                                                     const void* __restrict__ x, int act_bf16,
                                                     int32_t T, int32_t H, int32_t E,
                                                     double* __restrict__ z) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  double acc[kDecodeTokens];
#pragma unroll
  for (int n = 0; n < kDecodeTokens; ++n) acc[n] = 0.0;
  const float* wr = W + (int64_t)e * H;
  for (int h = lane * 4; h < H; h += 256) {
    const float4 w = *reinterpret_cast<const float4*>(wr + h);
#pragma unroll
    for (int n = 0; n < kDecodeTokens; ++n) {
      if (n < T) {
        const float4 v = load_x4(x, act_bf16, (int64_t)n * H + h);
        acc[n] = fma((double)w.x, (double)v.x, acc[n]);
        acc[n] = fma((double)w.y, (double)v.y, acc[n]);
        acc[n] = fma((double)w.z, (double)v.z, acc[n]);
        acc[n] = fma((double)w.w, (double)v.w, acc[n]);
      }
    }
  }
#pragma unroll
  for (int n = 0; n < kDecodeTokens; ++n) {
    if (n < T) {
      const double v = wave_sum(acc[n]);
      if (lane == 0) z[(int64_t)n * E + e] = v;
    }
  }
}

// Prefill shape: 64 tokens x 64 experts per block, fp64 FMA on LDS tiles.
constexpr int LG_BT = 64, LG_BE = 64, LG_BK = 16;
__global__ __launch_bounds__(256) void k_logits_gemm(const float* __restrict__ W,
                                                     const void* __restrict__ x, int act_bf16,
                                                     int32_t T, int32_t H, int32_t E,
                                                     double* __restrict__ z) {
  __shared__ float sx[LG_BK][LG_BT + 4];
  __shared__ float sw[LG_BK][LG_BE + 4];
  const int t0 = blockIdx.x * LG_BT, e0 = blockIdx.y * LG_BE;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  // each thread stages 4 consecutive k of one row of x and of W
  const int lr = threadIdx.x >> 2, lk = (threadIdx.x & 3) * 4;
  for (int k0 = 0; k0 < H; k0 += LG_BK) {
    {
      const int t = t0 + lr;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < T) v = load_x4(x, act_bf16, (int64_t)t * H + k0 + lk);
      sx[lk + 0][lr] = v.x;
      sx[lk + 1][lr] = v.y;
      sx[lk + 2][lr] = v.z;
      sx[lk + 3][lr] = v.w;
      const int e = e0 + lr;
      float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < E) w = *reinterpret_cast<const float4*>(W + (int64_t)e * H + k0 + lk);
      sw[lk + 0][lr] = w.x;
      sw[lk + 1][lr] = w.y;
      sw[lk + 2][lr] = w.z;
      sw[lk + 3][lr] = w.w;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < LG_BK; ++k) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = (double)sx[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = (double)sw[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) z[(int64_t)t * E + e] = acc[i][j];
    }
  }
}

hipError_t launch_router_logits(const float* w_router, const void* x, int act_bf16, int32_t T,
                                int32_t H, int32_t E, double* z, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (T <= kDecodeTokens) {
    hipLaunchKernelGGL(k_logits_gemv, dim3((E + 3) / 4), dim3(256), 0, s, w_router, x, act_bf16,
                       T, H, E, z);
  } else {
    dim3 grid((T + LG_BT - 1) / LG_BT, (E + LG_BE - 1) / LG_BE);
    hipLaunchKernelGGL(k_logits_gemm, grid, dim3(256), 0, s, w_router, x, act_bf16, T, H, E, z);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- selection
// One wave per token.  Lane l holds experts l*EPL .. l*EPL+EPL-1 (contiguous,
// so a group is a contiguous run of lanes' slots).  Every comparison prefers
// the larger score and, on equal scores, the lower index.

__device__ __forceinline__ bool beats(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Wave-wide best (value, index); every lane receives the winner.
__device__ __forceinline__ void wave_argbest(double& v, int& i) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const double ov = __shfl_xor(v, m, kWave);
    const int oi = __shfl_xor(i, m, kWave);
    if (beats(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

// Wave-wide two largest values (a >= b); lanes hold their local (a, b).
__device__ __forceinline__ void wave_top2(double& a, double& b) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const double oa = __shfl_xor(a, m, kWave);
    const double ob = __shfl_xor(b, m, kWave);
    const double hi = fmax(a, oa), lo = fmin(a, oa);
    b = fmax(lo, fmax(b, ob));
    a = hi;
  }
}

struct SelectParams {
  int32_t E, K, G, topk_group, softmax;
  float scaling;
};

template <int EPL>
__global__ __launch_bounds__(256) void k_select(SelectParams p, const double* __restrict__ z,
                                                const float* __restrict__ bias, int32_t T,
                                                int32_t* __restrict__ topk_idx,
                                                float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const double NEG = -INFINITY;
  const double* zt = z + (int64_t)t * p.E;
  double c[EPL], sv[EPL];
  bool open[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane * EPL + i;
    const bool ok = e < p.E;
    const double zv = ok ? zt[e] : 0.0;
    if (p.softmax) {
      sv[i] = zv;
      c[i] = ok ? zv : NEG;
    } else {
      const double s = 1.0 / (1.0 + exp(-zv));
      sv[i] = s;
      c[i] = ok ? s + (bias ? (double)bias[e] : 0.0) : NEG;
    }
    open[i] = ok;
  }

  if (!p.softmax && p.topk_group < p.G) {
    // group scores: sum of the two largest c in each contiguous group
    const int per = p.E / p.G;
    double my_gs = NEG;
    for (int g = 0; g < p.G; ++g) {
      double a = NEG, b = NEG;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        if (open[i] && e / per == g) {
          if (c[i] > a) {
            b = a;
            a = c[i];
          } else if (c[i] > b) {
            b = c[i];
          }
        }
      }
      wave_top2(a, b);
      if (lane == g) my_gs = (per == 1) ? a : a + b;
    }
    // keep the topk_group best groups
    uint64_t kept = 0;
    for (int r = 0; r < p.topk_group; ++r) {
      double v = ((kept >> lane) & 1ull) ? NEG : my_gs;
      int gi = lane < p.G && !((kept >> lane) & 1ull) ? lane : 0x7FFFFFFF;
      if (lane >= p.G) v = NEG;
      wave_argbest(v, gi);
      kept |= 1ull << gi;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane * EPL + i;
      if (open[i] && !((kept >> (e / per)) & 1ull)) open[i] = false;
    }
  }

  // top-k among open experts, in rank order
  int my_idx = 0;
  double my_s = 0.0, ssum = 0.0, z0 = 0.0;
  for (int j = 0; j < p.K; ++j) {
    double v = NEG;
    int bi = 0x7FFFFFFF;
    double bs = 0.0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane * EPL + i;
      if (open[i] && beats(c[i], e, v, bi)) {
        v = c[i];
        bi = e;
        bs = sv[i];
      }
    }
    // carry the winner's s along: reduce (v, bi), then fetch s from its owner
    double rv = v;
    int ri = bi;
    wave_argbest(rv, ri);
    const int owner = min(ri / EPL, kWave - 1);
    const double s_win = __shfl(bs, owner, kWave);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane * EPL + i == ri) open[i] = false;
    double contrib;
    if (p.softmax) {
      if (j == 0) z0 = s_win;
      contrib = exp(s_win - z0);
    } else {
      contrib = s_win;
    }
    ssum += contrib;   // sequential sum in rank order
    if (lane == j) {
      my_idx = ri;
      my_s = contrib;
    }
  }
  if (lane < p.K) {
    topk_idx[(int64_t)t * p.K + lane] = my_idx;
    topk_w[(int64_t)t * p.K + lane] = (float)(my_s / ssum * (double)p.scaling);
  }
}

hipError_t launch_router_select(const moe_layer_desc& d, const double* z, const float* bias,
                                int32_t T, int32_t* topk_idx, float* topk_w, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  SelectParams p;
  p.E = d.n_experts;
  p.K = d.top_k;
  p.softmax = d.router == MOE_ROUTER_SOFTMAX_TOPK;
  p.G = p.softmax ? 1 : d.n_group;
  p.topk_group = p.softmax ? 1 : d.topk_group;
  p.scaling = d.routed_scaling;
  const dim3 grid((T + 3) / 4), block(256);
  const int epl = (d.n_experts + 63) / 64;
  if (epl <= 1)
    hipLaunchKernelGGL(k_select<1>, grid, block, 0, s, p, z, bias, T, topk_idx, topk_w);
  else if (epl <= 2)
    hipLaunchKernelGGL(k_select<2>, grid, block, 0, s, p, z, bias, T, topk_idx, topk_w);
  else if (epl <= 4)
    hipLaunchKernelGGL(k_select<4>, grid, block, 0, s, p, z, bias, T, topk_idx, topk_w);
  else if (epl <= 8)
    hipLaunchKernelGGL(k_select<8>, grid, block, 0, s, p, z, bias, T, topk_idx, topk_w);
  else
    hipLaunchKernelGGL(k_select<16>, grid, block, 0, s, p, z, bias, T, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe
