// unpack.h -- the code unpacking of the expert kernels (gfx950), one
// definition each, shared by the decode GEMV (gemv_impl.h), the matrix-core
// grouped GEMM (k_ggemm.hip) and the dequantization hook (k_misc.hip), so that
// the hook's bit-exact check covers the very conversions the kernels run.
//
// Codes are packed int4 (two per byte, low nibble first), int2 (four per
// byte, element 4i + j in bits 2j..2j+1) or int8, two's complement, with one
// fp32 scale per output row ("colibri" README, "What's implemented": packed
// int4 / int2 with per-row scales, dequant-on-use).  The kernels read a code
// q in offset binary: q + 8 (int4, int8) or q + 2 (int2), a non-negative
// small integer whose byte, read as an OCP e4m3 float, is exactly
// (q + off) * 2^-9 for q + off in 0..15 (subnormals, then the first binade);
// the offset is removed later, from sums.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef float f32x2u __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4u __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2u __attribute__((ext_vector_type(2)));

// int4 for the fp32 kernels: the 8 codes of dword w as (q + 8) * 2^-9, even
// codes (bytes' low nibbles) in ql[0..3], odd ones in qh[0..3].
__device__ __forceinline__ void i4_unpack_f32(uint32_t w, float (&ql)[4], float (&qh)[4]) {
  const uint32_t lo = (w ^ 0x08080808u) & 0x0F0F0F0Fu;
  const uint32_t hi = ((w >> 4) ^ 0x08080808u) & 0x0F0F0F0Fu;
  const f32x2u l01 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
  const f32x2u l23 = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
  const f32x2u h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const f32x2u h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  ql[0] = l01.x;
  ql[1] = l01.y;
  ql[2] = l23.x;
  ql[3] = l23.y;
  qh[0] = h01.x;
  qh[1] = h01.y;
  qh[2] = h23.x;
  qh[3] = h23.y;
}

// int2 for the fp32 kernels: code jj of each byte of dword w (elements jj,
// 4 + jj, 8 + jj, 12 + jj) as (q + 2) * 2^-9.
__device__ __forceinline__ void i2_unpack_f32(uint32_t w, int jj, float (&q)[4]) {
  const uint32_t c = ((w ^ 0xAAAAAAAAu) >> (2 * jj)) & 0x03030303u;
  const f32x2u c01 = __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
  const f32x2u c23 = __builtin_amdgcn_cvt_pk_f32_fp8(c, true);
  q[0] = c01.x;
  q[1] = c01.y;
  q[2] = c23.x;
  q[3] = c23.y;
}

// int8 for the fp32 kernels: code b of dword w as (q + 8) / 512, one exact fma
// on the offset byte q + 128 -- for q in [-8, 7] the very operand the int4
// unpack yields, so int4 codes held in the int8 container give the same bits.
__device__ __forceinline__ float i8_unpack_f32(uint32_t w, int b) {
  return fmaf((float)(((w ^ 0x80808080u) >> (8 * b)) & 0xFFu), 1.0f / 512.0f, -120.0f / 512.0f);
}

// int4 for the matrix cores: the 8 codes of dword w as the exact bf16 values
// q + 8, in 4 registers of pairs: codes (0, 2), (4, 6), (1, 3), (5, 7).  The
// packed conversion to bf16 with the power-of-two scale 2^9 yields q + 8, two
// bytes per instruction.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t b, bool hi_word) {
  const bf16x2u v = hi_word ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 512.0f, true)
                            : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b, 512.0f, false);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4u i4_to_bf16(uint32_t w) {
  // mask and offset in one three-input bit operation each
  const uint32_t lo = (w & 0x0F0F0F0Fu) ^ 0x08080808u;          // codes 0, 2, 4, 6 in bytes 0..3
  const uint32_t hi = ((w >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;   // codes 1, 3, 5, 7
  u32x4u r;
  r.x = fp8x2_to_bf16x2(lo, false);
  r.y = fp8x2_to_bf16x2(lo, true);
  r.z = fp8x2_to_bf16x2(hi, false);
  r.w = fp8x2_to_bf16x2(hi, true);
  return r;
}

}  // namespace moe
