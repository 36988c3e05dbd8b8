// k_requant.hip -- FP8 (OCP E4M3, block scales) -> int4 per-row requantizer
// (gfx950): the step that produces the expert container from an FP8
// checkpoint ("colibri" README, "What's implemented": the offline converter
// dequantizes 128x128 block scales and requantizes to the engine's container).
//
// One block of 256 threads per row.  w = e4m3 * block scale is formed exactly
// in fp64 (an E4M3 value has 4 significant bits, the fp32 scale 24); the row's
// absolute maximum m gives the scale float(m / 7); codes are w / scale rounded
// to nearest even and clamped to [-7, 7], packed two per byte, low nibble
// first.  HBM-bound: each FP8 byte is read once and kept in registers for the
// second pass.
#include "moe_internal.h"

namespace moe {

constexpr int RQ_THREADS = 256;
constexpr int RQ_MAX_GROUPS = 4;   // 8-code groups per thread: cols <= 8192

__device__ __forceinline__ double block_max(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, kWave));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  return v;
}

__global__ __launch_bounds__(RQ_THREADS) void k_requant_fp8_int4(
    const uint8_t* __restrict__ fp8, const float* __restrict__ block_scales, int32_t cols,
    int32_t block, int32_t bcols, uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ double red[4];
  const int64_t r = blockIdx.x;
  const uint8_t* in = fp8 + r * cols;
  const float* bs = block_scales + (r / block) * bcols;
  const int groups = cols / 8;
  uint2 raw[RQ_MAX_GROUPS];
  float gsc[RQ_MAX_GROUPS];
  double m = 0.0;
#pragma unroll
  for (int i = 0; i < RQ_MAX_GROUPS; ++i) {
    const int g = threadIdx.x + i * RQ_THREADS;
    raw[i] = make_uint2(0u, 0u);
    gsc[i] = 0.f;
    if (g < groups) {
      raw[i] = *reinterpret_cast<const uint2*>(in + 8 * g);
      gsc[i] = bs[(8 * g) / block];   // block is a multiple of 8: one scale per group
      const uint32_t w2[2] = {raw[i].x, raw[i].y};
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const float2 lo = __builtin_bit_cast(float2, __builtin_amdgcn_cvt_pk_f32_fp8(w2[d], false));
        const float2 hi = __builtin_bit_cast(float2, __builtin_amdgcn_cvt_pk_f32_fp8(w2[d], true));
        const double s = (double)gsc[i];
        m = fmax(m, fabs((double)lo.x * s));
        m = fmax(m, fabs((double)lo.y * s));
        m = fmax(m, fabs((double)hi.x * s));
        m = fmax(m, fabs((double)hi.y * s));
      }
    }
  }
  m = block_max(m, red);
  const float sc = (float)(m / 7.0);
  if (threadIdx.x == 0) scales[r] = sc;
  const double sd = (double)sc;
  uint8_t* out = codes + r * (cols / 2);
#pragma unroll
  for (int i = 0; i < RQ_MAX_GROUPS; ++i) {
    const int g = threadIdx.x + i * RQ_THREADS;
    if (g >= groups) continue;
    const uint32_t w2[2] = {raw[i].x, raw[i].y};
    uint32_t packed = 0;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const float2 lo = __builtin_bit_cast(float2, __builtin_amdgcn_cvt_pk_f32_fp8(w2[d], false));
      const float2 hi = __builtin_bit_cast(float2, __builtin_amdgcn_cvt_pk_f32_fp8(w2[d], true));
      const float v4[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        double q = sc == 0.0f ? 0.0 : rint(((double)v4[k] * (double)gsc[i]) / sd);
        q = fmin(fmax(q, -7.0), 7.0);
        packed |= ((uint32_t)(int)q & 0xFu) << (4 * (4 * d + k));
      }
    }
    *reinterpret_cast<uint32_t*>(out + 4 * g) = packed;
  }
}

hipError_t launch_requant_fp8_int4(const uint8_t* fp8, const float* block_scales, int32_t rows,
                                   int32_t cols, int32_t block, uint8_t* codes, float* scales,
                                   hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int32_t bcols = (cols + block - 1) / block;
  hipLaunchKernelGGL(k_requant_fp8_int4, dim3((unsigned)rows), dim3(RQ_THREADS), 0, s, fp8,
                     block_scales, cols, block, bcols, codes, scales);
  return hipGetLastError();
}

bool requant_supported(int32_t cols, int32_t block) {
  return cols > 0 && cols % 8 == 0 && cols / 8 <= RQ_MAX_GROUPS * RQ_THREADS && block > 0 &&
         block % 8 == 0;
}

}  // namespace moe
