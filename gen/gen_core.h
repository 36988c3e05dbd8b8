/*
 * gen_core.h -- counter-based seeded draws for the synthetic inputs.
 *
 * Shared by the host generator (gen_host.c, built with gcc) and its device
 * twin (gen_dev.hip, built with hipcc), so that integer codes and per-row
 * scales come out bit-identical on both sides.  This file holds input
 * distributions only: it contains none of the MoE layer's arithmetic.
 *
 * Hash: the SplitMix64 output function (Steele, Lea & Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), used in
 * counter mode: draw(key, i) = mix64(key + golden * (i + 1)).
 *
 * The includer defines GEN_FN (e.g. "static inline" for C, or
 * "__host__ __device__ static inline" for HIP) before including.
 * All floating point here must be compiled with -ffp-contract=off so that the
 * host and the device twin round identically.
 */
#ifndef GEN_CORE_H
#define GEN_CORE_H

#include <stdint.h>

#ifndef GEN_FN
#define GEN_FN static inline
#endif

#define GEN_GOLDEN 0x9E3779B97F4A7C15ULL

/* Tensor ids that, with (seed, layer, expert), select an independent stream. */
enum {
  GEN_T_X = 0,          /* activations                                  */
  GEN_T_WROUTER = 1,    /* router weight [E][H]                         */
  GEN_T_BIAS = 2,       /* router correction bias [E]                   */
  GEN_T_GU_CODES = 3,   /* gate/up packed codes [2I][H/ppb]             */
  GEN_T_GU_SCALES = 4,  /* gate/up per-row scales [2I]                  */
  GEN_T_DN_CODES = 5,   /* down packed codes [H][I/ppb]                 */
  GEN_T_DN_SCALES = 6,  /* down per-row scales [H]                      */
  GEN_T_GU_BF16 = 7,    /* gate/up bf16 weights [2I][H]                 */
  GEN_T_DN_BF16 = 8,    /* down bf16 weights [H][I]                     */
  GEN_T_ZIPF_PERM = 9,  /* expert popularity permutation                */
  GEN_T_GU_I8 = 10,     /* gate/up int8 codes [2I][H]                   */
  GEN_T_DN_I8 = 11,     /* down int8 codes [H][I]                       */
  GEN_T_GU_BYTES = 12,  /* gate/up codes as uniform bytes (full range)  */
  GEN_T_DN_BYTES = 13   /* down codes as uniform bytes (full range)     */
};

GEN_FN uint64_t gen_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Stream key for one (seed, layer, tensor, expert) tuple. */
GEN_FN uint64_t gen_key(uint64_t seed, uint64_t layer, uint64_t tensor, uint64_t expert) {
  uint64_t k = gen_mix64(GEN_GOLDEN * (seed + 1));
  k = gen_mix64(k + GEN_GOLDEN * (layer + 1));
  k = gen_mix64(k + GEN_GOLDEN * (tensor + 1));
  k = gen_mix64(k + GEN_GOLDEN * (expert + 1));
  return k;
}

GEN_FN uint64_t gen_draw(uint64_t key, uint64_t i) {
  return gen_mix64(key + GEN_GOLDEN * (i + 1));
}

/* Uniform on [0,1) with 24 random bits: exactly representable in float. */
GEN_FN double gen_u24(uint64_t r) {
  return (double)(r >> 40) * (1.0 / 16777216.0);
}

/* Integer uniform on {0, ..., n-1} from 32 random bits (multiply-shift). */
GEN_FN uint32_t gen_below(uint32_t r32, uint32_t n) {
  return (uint32_t)(((uint64_t)r32 * (uint64_t)n) >> 32);
}

/* One packed byte of symmetric int4 codes, each uniform on {-7, ..., 7}:
 * element 2i in bits 0-3, element 2i+1 in bits 4-7, two's complement. */
GEN_FN uint8_t gen_int4_byte(uint64_t key, uint64_t byte_index) {
  uint64_t r = gen_draw(key, byte_index);
  int lo = (int)gen_below((uint32_t)(r & 0xFFFFFFFFu), 15u) - 7;
  int hi = (int)gen_below((uint32_t)(r >> 32), 15u) - 7;
  return (uint8_t)(((unsigned)lo & 0xFu) | (((unsigned)hi & 0xFu) << 4));
}

/* Two int8 codes, each uniform on {-127, ..., 127}: element 2i in the low
 * byte, element 2i+1 in the high byte, two's complement. */
GEN_FN uint16_t gen_int8_pair(uint64_t key, uint64_t pair_index) {
  uint64_t r = gen_draw(key, pair_index);
  int lo = (int)gen_below((uint32_t)(r & 0xFFFFFFFFu), 255u) - 127;
  int hi = (int)gen_below((uint32_t)(r >> 32), 255u) - 127;
  return (uint16_t)(((unsigned)lo & 0xFFu) | (((unsigned)hi & 0xFFu) << 8));
}

/* A uniform byte: byte i % 8 of draw i / 8.  As packed codes it covers the
 * whole two's-complement range of every container: int4 [-8, 7], int2
 * [-2, 1], int8 [-128, 127]. */
GEN_FN uint8_t gen_byte(uint64_t key, uint64_t i) {
  return (uint8_t)(gen_draw(key, i >> 3) >> (8 * (i & 7)));
}

/* Signed value of nibble j (0 or 1) of a packed int4 byte. */
GEN_FN int gen_nibble(uint8_t b, int j) {
  int v = (b >> (4 * j)) & 0xF;
  return v >= 8 ? v - 16 : v;
}

/* Per-row scale: (lo + width * u) * mult, evaluated in double, rounded once
 * to float.  mult is computed by the caller (host) and passed in. */
GEN_FN float gen_scale(uint64_t key, uint64_t row, double lo, double width, double mult) {
  double u = gen_u24(gen_draw(key, row));
  double v = lo + width * u;
  v = v * mult;
  return (float)v;
}

/* int2 code of an int4 code q given the row's absolute maximum m >= 1:
 * round-to-nearest-even of q/m, clamped to [-1, 1], in integers:
 * |q/m| > 1/2 -> sign(q), |q/m| <= 1/2 -> 0 (the tie goes to even 0). */
GEN_FN int gen_int2_of_int4(int q, int m) {
  int a = q < 0 ? -q : q;
  if (2 * a > m) return q < 0 ? -1 : 1;
  return 0;
}

#endif /* GEN_CORE_H */
