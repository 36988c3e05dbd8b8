/*
 * gen_dev.hip -- device twin of the seeded generator for the large integer
 * tensors (packed int4 codes, their per-row scales, and the derived int2
 * variant), so that tens of GB of expert weights can be produced in place in
 * HBM.  Uses the same gen_core.h functions as the host generator, so every
 * byte and every scale is bit-identical to gen_host.c's.
 *
 * Input preparation only: nothing here is part of the MoE layer.
 * Build: hipcc --offload-arch=gfx950 -O2 -ffp-contract=off -shared -fPIC.
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#define GEN_FN __host__ __device__ static inline
#include "gen_core.h"

__global__ void k_fill_int4_set(uint8_t* dst, int64_t stride, int64_t bytes_per_expert,
                                uint64_t seed, int32_t layer, int32_t tensor, int32_t expert0) {
  const int e = blockIdx.y;
  const uint64_t key = gen_key(seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)(expert0 + e));
  uint8_t* out = dst + (int64_t)e * stride;
  /* 4 bytes per thread per step: one 32-bit store */
  const int64_t n4 = bytes_per_expert / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    uint32_t w = 0;
    for (int b = 0; b < 4; ++b) w |= (uint32_t)gen_int4_byte(key, (uint64_t)(4 * i + b)) << (8 * b);
    reinterpret_cast<uint32_t*>(out)[i] = w;
  }
  const int64_t tail0 = n4 * 4;
  if (blockIdx.x == 0)
    for (int64_t i = tail0 + threadIdx.x; i < bytes_per_expert; i += blockDim.x)
      out[i] = gen_int4_byte(key, (uint64_t)i);
}

__global__ void k_fill_int8_set(uint8_t* dst, int64_t stride, int64_t bytes_per_expert,
                                uint64_t seed, int32_t layer, int32_t tensor, int32_t expert0) {
  const int e = blockIdx.y;
  const uint64_t key = gen_key(seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)(expert0 + e));
  uint8_t* out = dst + (int64_t)e * stride;
  /* 4 bytes (two pairs) per thread per step: one 32-bit store */
  const int64_t n4 = bytes_per_expert / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t w = (uint32_t)gen_int8_pair(key, (uint64_t)(2 * i)) |
                       ((uint32_t)gen_int8_pair(key, (uint64_t)(2 * i + 1)) << 16);
    reinterpret_cast<uint32_t*>(out)[i] = w;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && (bytes_per_expert & 3)) {
    const uint16_t v = gen_int8_pair(key, (uint64_t)(2 * n4));
    out[4 * n4] = (uint8_t)(v & 0xFFu);
    out[4 * n4 + 1] = (uint8_t)(v >> 8);
  }
}

__global__ void k_fill_scales_set(uint8_t* dst, int64_t stride, int64_t rows, uint64_t seed,
                                  int32_t layer, int32_t tensor, int32_t expert0, double lo,
                                  double width, double mult) {
  const int e = blockIdx.y;
  const uint64_t key = gen_key(seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)(expert0 + e));
  float* out = reinterpret_cast<float*>(dst + (int64_t)e * stride);
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < rows;
       r += (int64_t)gridDim.x * blockDim.x)
    out[r] = gen_scale(key, (uint64_t)r, lo, width, mult);
}

/* One block per (row, expert): int2 variant of one int4 row (see gen_host.c). */
__global__ void k_int2_from_int4_set(const uint8_t* codes4, int64_t stride4, const uint8_t* s4,
                                     int64_t s4_stride, uint8_t* codes2, int64_t stride2,
                                     uint8_t* s2, int64_t s2_stride, int64_t rows, int64_t cols) {
  __shared__ int red[256];
  const int64_t r = blockIdx.x;
  const int e = blockIdx.y;
  const uint8_t* src = codes4 + (int64_t)e * stride4 + r * (cols / 2);
  uint8_t* dst = codes2 + (int64_t)e * stride2 + r * (cols / 4);
  int m = 0;
  for (int64_t b = threadIdx.x; b < cols / 2; b += blockDim.x) {
    for (int j = 0; j < 2; ++j) {
      int q = gen_nibble(src[b], j);
      int a = q < 0 ? -q : q;
      m = a > m ? a : m;
    }
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = blockDim.x / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  m = red[0];
  if (threadIdx.x == 0) {
    const float sv = reinterpret_cast<const float*>(s4 + (int64_t)e * s4_stride)[r];
    reinterpret_cast<float*>(s2 + (int64_t)e * s2_stride)[r] =
        m == 0 ? sv : (float)((double)sv * (double)m);
  }
  for (int64_t b = threadIdx.x; b < cols / 4; b += blockDim.x) {
    unsigned byte = 0;
    for (int j = 0; j < 4; ++j) {
      int64_t c = 4 * b + j;
      int q = gen_nibble(src[c >> 1], (int)(c & 1));
      int q2 = m == 0 ? 0 : gen_int2_of_int4(q, m);
      byte |= ((unsigned)q2 & 3u) << (2 * j);
    }
    dst[b] = (uint8_t)byte;
  }
}

static int grid_for(int64_t n, int per_block) {
  int64_t g = (n + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > 65535) g = 65535;
  return (int)g;
}

extern "C" {

/* Fill n_experts packed-int4 matrices of bytes_per_expert bytes each, the
 * e-th at dst + e*stride, with the stream of expert (expert0 + e). */
int gen_dev_fill_int4_set(void* dst, int64_t stride, int32_t n_experts, int64_t bytes_per_expert,
                          uint64_t seed, int32_t layer, int32_t tensor, int32_t expert0,
                          hipStream_t s) {
  if (n_experts <= 0 || bytes_per_expert <= 0) return 0;
  dim3 grid(grid_for(bytes_per_expert / 4, 256 * 4), n_experts);
  hipLaunchKernelGGL(k_fill_int4_set, grid, dim3(256), 0, s, (uint8_t*)dst, stride,
                     bytes_per_expert, seed, layer, tensor, expert0);
  return (int)hipGetLastError();
}

/* Fill n_experts int8 matrices of bytes_per_expert (even) bytes each, the
 * e-th at dst + e*stride, with the stream of expert (expert0 + e). */
int gen_dev_fill_int8_set(void* dst, int64_t stride, int32_t n_experts, int64_t bytes_per_expert,
                          uint64_t seed, int32_t layer, int32_t tensor, int32_t expert0,
                          hipStream_t s) {
  if (bytes_per_expert & 1) return (int)hipErrorInvalidValue;   /* whole pairs only */
  if (n_experts <= 0 || bytes_per_expert <= 0) return 0;
  dim3 grid(grid_for(bytes_per_expert / 4, 256 * 4), n_experts);
  hipLaunchKernelGGL(k_fill_int8_set, grid, dim3(256), 0, s, (uint8_t*)dst, stride,
                     bytes_per_expert, seed, layer, tensor, expert0);
  return (int)hipGetLastError();
}

int gen_dev_fill_scales_set(void* dst, int64_t stride, int32_t n_experts, int64_t rows,
                            uint64_t seed, int32_t layer, int32_t tensor, int32_t expert0,
                            double lo, double width, double mult, hipStream_t s) {
  if (n_experts <= 0 || rows <= 0) return 0;
  dim3 grid(grid_for(rows, 256), n_experts);
  hipLaunchKernelGGL(k_fill_scales_set, grid, dim3(256), 0, s, (uint8_t*)dst, stride, rows, seed,
                     layer, tensor, expert0, lo, width, mult);
  return (int)hipGetLastError();
}

int gen_dev_int2_from_int4_set(const void* codes4, int64_t stride4, const void* s4,
                               int64_t s4_stride, void* codes2, int64_t stride2, void* s2,
                               int64_t s2_stride, int32_t n_experts, int64_t rows, int64_t cols,
                               hipStream_t s) {
  if (n_experts <= 0 || rows <= 0) return 0;
  if (rows > 2147483647LL || (cols % 4) != 0) return 1;
  dim3 grid((unsigned)rows, n_experts);
  hipLaunchKernelGGL(k_int2_from_int4_set, grid, dim3(256), 0, s, (const uint8_t*)codes4,
                     stride4, (const uint8_t*)s4, s4_stride, (uint8_t*)codes2, stride2,
                     (uint8_t*)s2, s2_stride, rows, cols);
  return (int)hipGetLastError();
}

}  // extern "C"
