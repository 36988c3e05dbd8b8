/*
 * gen_host.c -- host fill routines for the seeded synthetic inputs.
 *
 * Exposed with a plain C ABI (loaded from Python with ctypes).  Every value is
 * a pure function of (seed, layer, tensor, expert, index); OpenMP only splits
 * the index range, so results do not depend on the thread count.
 *
 * Distributions (the reading of each workload's description):
 *   int4 codes  uniform on {-7..7}, two per byte, low nibble first;
 *   scales      (lo + width * U[0,1)) * mult, rounded once to float;
 *   normals     Box-Muller in double from two 53-bit uniforms, times std,
 *               rounded to float (and then to bf16 where asked).
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GEN_FN static inline
#include "gen_core.h"

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  if ((b & 0x7F800000u) == 0x7F800000u) return (uint16_t)(b >> 16); /* inf/nan: truncate */
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

static double normal_at(uint64_t key, uint64_t i) {
  uint64_t r1 = gen_draw(key, 2 * i);
  uint64_t r2 = gen_draw(key, 2 * i + 1);
  double u1 = (double)((r1 >> 11) + 1) * (1.0 / 9007199254740992.0); /* (0,1] */
  double u2 = (double)(r2 >> 11) * (1.0 / 9007199254740992.0);       /* [0,1) */
  const double two_pi = 6.283185307179586476925286766559;
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* Packed int4 codes of one matrix of one expert: n_bytes bytes. */
void gen_fill_int4(uint8_t* dst, uint64_t seed, int32_t layer, int32_t tensor, int32_t expert,
                   int64_t n_bytes) {
  uint64_t key = gen_key(seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)expert);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_bytes; ++i) dst[i] = gen_int4_byte(key, (uint64_t)i);
}

/* Uniform bytes (packed codes over their whole range): n_bytes bytes. */
void gen_fill_bytes(uint8_t* dst, uint64_t seed, int32_t layer, int32_t tensor, int32_t expert,
                    int64_t n_bytes) {
  uint64_t key = gen_key(seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)expert);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_bytes; ++i) dst[i] = gen_byte(key, (uint64_t)i);
}

/* int8 codes of one matrix of one expert: n_bytes bytes (even). */
void gen_fill_int8(uint8_t* dst, uint64_t seed, int32_t layer, int32_t tensor, int32_t expert,
                   int64_t n_bytes) {
  uint64_t key = gen_key(seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)expert);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_bytes / 2; ++i) {
    uint16_t v = gen_int8_pair(key, (uint64_t)i);
    dst[2 * i] = (uint8_t)(v & 0xFFu);
    dst[2 * i + 1] = (uint8_t)(v >> 8);
  }
}

/* Per-row scales of one matrix of one expert. */
void gen_fill_scales(float* dst, uint64_t seed, int32_t layer, int32_t tensor, int32_t expert,
                     int64_t rows, double lo, double width, double mult) {
  uint64_t key = gen_key(seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)expert);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) dst[r] = gen_scale(key, (uint64_t)r, lo, width, mult);
}

void gen_fill_normal_f32(float* dst, int64_t n, uint64_t seed, int32_t layer, int32_t tensor,
                         int32_t expert, double std) {
  uint64_t key = gen_key(seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)expert);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) dst[i] = (float)(normal_at(key, (uint64_t)i) * std);
}

void gen_fill_normal_bf16(uint16_t* dst, int64_t n, uint64_t seed, int32_t layer, int32_t tensor,
                          int32_t expert, double std) {
  uint64_t key = gen_key(seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)expert);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) dst[i] = f32_to_bf16_rne((float)(normal_at(key, (uint64_t)i) * std));
}

/* Uniform 64-bit draws (used for seeded permutations). */
void gen_fill_u64(uint64_t* dst, int64_t n, uint64_t seed, int32_t layer, int32_t tensor,
                  int32_t expert) {
  uint64_t key = gen_key(seed, (uint64_t)layer, (uint64_t)tensor, (uint64_t)expert);
  for (int64_t i = 0; i < n; ++i) dst[i] = gen_draw(key, (uint64_t)i);
}

/* The int2 variant of an int4 matrix [rows][cols] (cols even, multiple of 4):
 * per row m = max |q4| (m = 0: all codes 0, scale kept), s2 = float(s4 * m),
 * q2 = round-half-even(q4 / m) clamped to [-1, 1]; four codes per byte, element
 * 4i+j in bits 2j..2j+1, two's complement. */
void gen_int2_from_int4(const uint8_t* codes4, const float* s4, int64_t rows, int64_t cols,
                        uint8_t* codes2, float* s2) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint8_t* src = codes4 + r * (cols / 2);
    uint8_t* dst = codes2 + r * (cols / 4);
    int m = 0;
    for (int64_t c = 0; c < cols; ++c) {
      int q = gen_nibble(src[c >> 1], (int)(c & 1));
      int a = q < 0 ? -q : q;
      if (a > m) m = a;
    }
    s2[r] = m == 0 ? s4[r] : (float)((double)s4[r] * (double)m);
    for (int64_t b = 0; b < cols / 4; ++b) {
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
}
