// k_misc.hip -- weighted combine of the routed experts plus the shared expert,
// and the dequantization test hook (gfx950).
#include "moe_internal.h"
#include "unpack.h"

namespace moe {

// out[t][o] = sum_j w[t][j] * Y[t*K + j][o] (j ascending, slots with index
// -1 skipped) + S[t][o]
// ("colibri" README, "What's implemented": routed_scaling_factor-weighted
// combine with a shared expert; the scaling is already inside w).
// With a residual: y_copy (optional) = the MoE output, out = residual + it.
// residual and out may be the same buffer (a stack adds each layer into the
// running hidden state in place): each thread reads its four residual values
// before it writes the same four outputs, and neither pointer is restrict.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ Y,
                                                 const int32_t* __restrict__ topk_idx,
                                                 const float* __restrict__ topk_w,
                                                 const float* __restrict__ S, int32_t K,
                                                 int32_t H, const float* residual,
                                                 float* out,
                                                 float* __restrict__ y_copy) {
  const int64_t t = blockIdx.y;
  const int o = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (o >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < K; ++j) {
    if (topk_idx[t * K + j] < 0) continue;   // dropped by adaptive top-p: no Y row
    const float w = topk_w[t * K + j];
    const float4 y = *reinterpret_cast<const float4*>(Y + (t * K + j) * H + o);
    acc.x = fmaf(w, y.x, acc.x);
    acc.y = fmaf(w, y.y, acc.y);
    acc.z = fmaf(w, y.z, acc.z);
    acc.w = fmaf(w, y.w, acc.w);
  }
  if (S) {
    const float4 sv = *reinterpret_cast<const float4*>(S + t * H + o);
    acc.x += sv.x;
    acc.y += sv.y;
    acc.z += sv.z;
    acc.w += sv.w;
  }
  if (residual) {
    if (y_copy) *reinterpret_cast<float4*>(y_copy + t * H + o) = acc;
    const float4 r = *reinterpret_cast<const float4*>(residual + t * H + o);
    acc.x += r.x;
    acc.y += r.y;
    acc.z += r.z;
    acc.w += r.w;
  }
  *reinterpret_cast<float4*>(out + t * H + o) = acc;
}

// SwiGLU over fp32 gate/up rows: h[t][c] = bf16(silu(g) * u) with
// g = GU[t][c], u = GU[t][Is + c] (the dense shared-expert path's gate/up
// output, "iliria" README, "What's implemented": SwiGLU over one
// activation); hp (nullable) receives h before rounding.
__global__ __launch_bounds__(256) void k_swiglu_rows(const float* __restrict__ GU, int32_t T,
                                                     int32_t Is, uint16_t* __restrict__ h,
                                                     float* __restrict__ hp) {
  const int64_t n = (int64_t)T * Is;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t t = i / Is, c = i - t * Is;
    const float g = GU[t * 2 * Is + c], u = GU[t * 2 * Is + Is + c];
    const float hv = g / (1.0f + expf(-g)) * u;
    h[i] = f32_to_bf16_bits(hv);
    if (hp) hp[i] = hv;
  }
}

hipError_t launch_swiglu_rows(const float* gu, int32_t T, int32_t Is, uint16_t* h, float* hp,
                              hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int64_t n = (int64_t)T * Is;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_swiglu_rows, dim3((unsigned)blocks), dim3(256), 0, s, gu, T, Is, h, hp);
  return hipGetLastError();
}

hipError_t launch_combine(const float* Y, const int32_t* topk_idx, const float* topk_w,
                          const float* S, int32_t T, int32_t K, int32_t H, const float* residual,
                          float* out, float* y_copy, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((H / 4 + 255) / 256, T);
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, s, Y, topk_idx, topk_w, S, K, H, residual,
                     out, y_copy);
  return hipGetLastError();
}

// Dequantized weights: out[r][c] = float(q) * scale[row0 + r] (one rounded
// fp32 multiply); out_bf16 = bf16 bits of q (exact for |q| <= 256).  The codes
// go through the kernels' own unpacking (unpack.h): q comes from the operand
// the fp32 (GEMV) kernels read, (q + off) * 2^-9 for int4 and int2, (q + 8) /
// 512 for int8, and for int4 the bf16 code from the matrix-core operand
// q + 8; removing the offsets is exact.
__global__ __launch_bounds__(256) void k_dequant(int dtype, const uint8_t* __restrict__ codes,
                                                 const float* __restrict__ scales, int32_t cols,
                                                 int32_t row0, int32_t n_rows,
                                                 float* __restrict__ out,
                                                 uint16_t* __restrict__ out_bf16) {
  const int64_t n = (int64_t)n_rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = row0 + i / cols;
    const int64_t c = i % cols;
    if (dtype == MOE_BF16) {
      const uint16_t b = reinterpret_cast<const uint16_t*>(codes)[r * cols + c];
      out[i] = bf16_bits_to_f32(b);
      continue;
    }
    float q;
    float qb = 0.f;   // int4: the code from the matrix-core operand
    if (dtype == MOE_I4) {
      // the dword holding elements 8 (c / 8) .. + 7 (rows are whole bytes;
      // the dword is read bytewise, as a row need not be 4-byte aligned)
      const int64_t b0 = r * (cols / 2) + (c / 8) * 4;
      const int64_t rb = r * (cols / 2) + cols / 2;
      uint32_t w = 0;
      for (int k = 0; k < 4; ++k)
        if (b0 + k < rb) w |= (uint32_t)codes[b0 + k] << (8 * k);
      const int e = (int)(c & 7);
      float ql[4], qh[4];
      i4_unpack_f32(w, ql, qh);
      q = fmaf((e & 1) ? qh[e >> 1] : ql[e >> 1], 512.0f, -8.0f);
      const u32x4u ob = i4_to_bf16(w);
      // registers hold codes (0, 2), (4, 6), (1, 3), (5, 7)
      const uint32_t reg = (e & 1) ? ((e >> 2) ? ob.w : ob.z) : ((e >> 2) ? ob.y : ob.x);
      const int half = (e >> 1) & 1;
      qb = bf16_bits_to_f32(half ? reg >> 16 : reg & 0xFFFFu) - 8.0f;
    } else if (dtype == MOE_I2) {
      const int64_t b0 = r * (cols / 4) + (c / 16) * 4;
      const int64_t rb = r * (cols / 4) + cols / 4;
      uint32_t w = 0;
      for (int k = 0; k < 4; ++k)
        if (b0 + k < rb) w |= (uint32_t)codes[b0 + k] << (8 * k);
      const int e = (int)(c & 15);
      float v[4];
      i2_unpack_f32(w, e & 3, v);
      q = fmaf(v[e >> 2], 512.0f, -2.0f);
    } else {
      const int64_t b0 = r * (int64_t)cols + (c / 4) * 4;
      const int64_t rb = r * (int64_t)cols + cols;
      uint32_t w = 0;
      for (int k = 0; k < 4; ++k)
        if (b0 + k < rb) w |= (uint32_t)codes[b0 + k] << (8 * k);
      q = fmaf(i8_unpack_f32(w, (int)(c & 3)), 512.0f, -8.0f);
    }
    out[i] = __fmul_rn(q, scales[r]);
    if (out_bf16) out_bf16[i] = f32_to_bf16_bits(dtype == MOE_I4 ? qb : q);
  }
}

hipError_t launch_dequant(int dtype, const void* codes, const float* scales, int32_t cols,
                          int32_t row0, int32_t n_rows, float* out, uint16_t* out_bf16,
                          hipStream_t s) {
  const int64_t n = (int64_t)n_rows * cols;
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)blocks), dim3(256), 0, s, dtype,
                     reinterpret_cast<const uint8_t*>(codes), scales, cols, row0, n_rows, out,
                     out_bf16);
  return hipGetLastError();
}

// Sliced copies of activation rows (layout in moe_internal.h): every thread
// moves one 16-byte piece per format; the writes are coalesced, the reads
// gather the piece's P consecutive activations.
__global__ __launch_bounds__(256) void k_slice_rows(const uint8_t* __restrict__ x, int32_t ab,
                                                    int32_t K, int32_t T, int32_t epg_a,
                                                    uint8_t* __restrict__ dst_a, int32_t epg_b,
                                                    uint8_t* __restrict__ dst_b) {
  const int64_t pieces = (int64_t)K * ab / 16;
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = blockIdx.y;
  if (p >= pieces || t >= T) return;
  const int64_t row = t * K * ab;
  if (dst_a && epg_a > 0) slice_piece(x + row, dst_a + row, p, epg_a, ab);
  if (dst_b && epg_b > 0) slice_piece(x + row, dst_b + row, p, epg_b, ab);
}

hipError_t launch_slice_rows(const void* x, int act_bf16, int32_t T, int32_t K, int32_t epg_a,
                             void* dst_a, int32_t epg_b, void* dst_b, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int ab = act_bf16 ? 2 : 4;
  const int64_t pieces = (int64_t)K * ab / 16;
  const dim3 grid((unsigned)((pieces + 255) / 256), (unsigned)T);
  hipLaunchKernelGGL(k_slice_rows, grid, dim3(256), 0, s, reinterpret_cast<const uint8_t*>(x), ab,
                     K, T, epg_a, reinterpret_cast<uint8_t*>(dst_a), epg_b,
                     reinterpret_cast<uint8_t*>(dst_b));
  return hipGetLastError();
}

}  // namespace moe
