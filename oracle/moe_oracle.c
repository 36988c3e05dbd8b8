/*
 * moe_oracle.c -- plain, slow, obviously correct CPU oracle of the routed MoE
 * layer forward.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
 * CPU-baseline leg load it; the product path never does.  It shares no code
 * with the HIP library.
 *
 * Method, as the pages describe it:
 *   - "colibri" README (Tiny engine, immense model), section "What's
 *     implemented": a DeepSeek-V3-style sigmoid router (noaux_tc,
 *     routed_scaling_factor) with a shared expert; quantized experts in packed
 *     int4 / packed int2 with per-row scales, dequantized on use; batch-union
 *     MoE, where each unique expert of a batch is applied to every position
 *     routed to it.
 *   - "iliria" README, section "What's implemented": routed-expert SwiGLU;
 *     gate and up fused over one activation.
 *   - "Glacial" page, section "Important invariants": greedy selection is the
 *     first maximum (our tie rule: the lowest index wins every comparison).
 *   - "muse-glimmer-intel-serve" page, introduction: a deterministic float64
 *     CPU implementation defines the function; low-precision kernels are gated
 *     against it.
 *   - "Local run: open-1b on one Arc B580", section "Tensor mapping": casts
 *     round to nearest, ties to even (our rule for every narrowing cast).
 *
 * Arithmetic: every input widens exactly to double.  A code times its
 * float scale is exact in double (at most 8 + 24 significant bits), and that
 * times a float activation is exact too (at most 52 bits); sums run in index
 * order in double.  The only roundings to narrower types are the ones the
 * layer defines: topk weights to float, h to bf16 when activations are bf16,
 * RMSNorm output and residual stream to float.
 *
 * Parity status (what pins each function; the tests under tests/ hold them):
 *   orc_decode_codes     exhaustive round trip over all bytes (int4, int2,
 *                        int8); worked bytes; int4 codes re-packed as int8
 *                        decode to the same values.
 *   orc_dequant_rows     integer and power-of-two scale cases, exact.
 *   orc_logits           one-hot and small-integer inputs (exact matmul).
 *   orc_select           brute-force subset search on small E, exact ties,
 *                        reductions to plain top-k, closed-form weights;
 *                        adaptive top-p: a worked example with exact masses,
 *                        off values equal the plain router, kept set a prefix
 *                        with minimal sufficient mass, weights proportional
 *                        and summing to the scaling, monotone in top_p.
 *   orc_route            = orc_logits + orc_select.
 *   orc_bucket           numpy stable argsort; permutation invariants;
 *                        dropped slots (-1) left out, inverse -1.
 *   orc_layer_band       a test tolerance, not part of the layer: zero for f32
 *                        activations and for a zero window, monotone in the
 *                        window, and equal to the sum over every h at the
 *                        widest window (checked against orc_dequant_rows).
 *   orc_expert_ffn       worked H=2,I=1 example; integer-matrix case against
 *                        numpy matmul and scipy's logistic; scale factoring.
 *   orc_layer_forward    dense evaluation of all experts; batch-union equals
 *                        per-token; x=0; E=1,k=1; token permutation; the
 *                        int8 container of int4 codes gives the same bits;
 *                        with top-p, the sum over the kept experts.
 *   orc_rmsnorm          closed-form rms of the output.
 *   orc_decode_e4m3      every byte against torch's float8_e4m3fn; worked
 *                        values (0, 2^-9, 2^-6, 1, 448, NaN).
 *   orc_requant_fp8_int4 exact round trips of integer multiples of a scale;
 *                        the row's absmax maps to +-7; |q*s - w| <= s/2; ties
 *                        to even; per-block scales; zero rows.
 *   orc_residual_add     f32 addition, exact cases.
 *
 * Build: gcc -O2 -fopenmp -fno-fast-math -ffp-contract=off -shared -fPIC.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- casts -- */

static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* float -> bf16, round to nearest, ties to even. */
static uint16_t float_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)(u >> 16);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

static double x_at(const void* x, int bf16, int64_t i) {
  if (bf16) return bf16_to_double(((const uint16_t*)x)[i]);
  return (double)((const float*)x)[i];
}

/* --------------------------------------------------------------- codecs -- */

/* Packed int4: element i sits in byte i/2, low nibble first (even elements in
 * bits 0-3), as a two's-complement nibble.  Packed int2: element i sits in byte
 * i/4 at bits 2*(i%4)..2*(i%4)+1, two's complement.  int8: element i is byte i,
 * two's complement.  ("colibri" README, "What's implemented": packed int4 /
 * packed int2 containers next to the int8 container they were validated
 * against.) */
static int code_at(int32_t dtype, const uint8_t* p, int64_t i) {
  if (dtype == ORC_I4) {
    int v = (p[i / 2] >> (4 * (int)(i % 2))) & 0xF;
    return v >= 8 ? v - 16 : v;
  } else if (dtype == ORC_I2) {
    int v = (p[i / 4] >> (2 * (int)(i % 4))) & 0x3;
    return v >= 2 ? v - 4 : v;
  } else {
    int v = p[i];
    return v >= 128 ? v - 256 : v;
  }
}

static int is_code_dtype(int32_t dtype) {
  return dtype == ORC_I4 || dtype == ORC_I2 || dtype == ORC_I8;
}

int orc_decode_codes(int32_t dtype, const uint8_t* packed, int64_t n, int8_t* out) {
  if (!is_code_dtype(dtype)) return ORC_EINVAL;
  for (int64_t i = 0; i < n; ++i) out[i] = (int8_t)code_at(dtype, packed, i);
  return ORC_OK;
}

static int64_t row_bytes(int32_t dtype, int64_t cols) {
  if (dtype == ORC_I4) return cols / 2;
  if (dtype == ORC_I2) return cols / 4;
  if (dtype == ORC_I8) return cols;
  return cols * 2;
}

/* Weight element (r, c) of a matrix, as an exact double: code * row scale, or
 * the bf16 value.  Dequant-on-use with per-row scales ("colibri" README). */
static double weight_at(int32_t dtype, const void* m, const float* scale, int64_t cols, int64_t r,
                        int64_t c) {
  if (dtype == ORC_BF16) return bf16_to_double(((const uint16_t*)m)[r * cols + c]);
  const uint8_t* row = (const uint8_t*)m + r * row_bytes(dtype, cols);
  return (double)code_at(dtype, row, c) * (double)scale[r];
}

/* The float dequantized weight: one IEEE float multiply of the code by its row
 * scale, round to nearest even. */
int orc_dequant_rows(int32_t dtype, const void* codes, const float* scales, int64_t cols,
                     int64_t row0, int64_t n_rows, float* out) {
  if (!is_code_dtype(dtype) && dtype != ORC_BF16) return ORC_EINVAL;
  for (int64_t r = 0; r < n_rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      if (dtype == ORC_BF16) {
        out[r * cols + c] = (float)bf16_to_double(((const uint16_t*)codes)[(row0 + r) * cols + c]);
      } else {
        const uint8_t* row = (const uint8_t*)codes + (row0 + r) * row_bytes(dtype, cols);
        float q = (float)code_at(dtype, row, c);
        float s = scales[row0 + r];
        out[r * cols + c] = q * s;
      }
    }
  }
  return ORC_OK;
}

/* --------------------------------------------------------------- router -- */

static int desc_ok(const orc_desc* d) {
  if (!d || d->hidden <= 0 || d->inter <= 0 || d->n_experts <= 0) return 0;
  if (d->top_k <= 0 || d->top_k > d->n_experts) return 0;
  if (d->router == ORC_ROUTER_SIGMOID_NOAUX_TC) {
    if (d->n_group <= 0 || d->n_experts % d->n_group != 0) return 0;
    if (d->topk_group <= 0 || d->topk_group > d->n_group) return 0;
    if ((int64_t)d->topk_group * (d->n_experts / d->n_group) < d->top_k) return 0;
  } else if (d->router != ORC_ROUTER_SOFTMAX_TOPK) {
    return 0;
  }
  if (!(d->top_p >= 0.0)) return 0;   /* also rejects NaN */
  return 1;
}

/* Router logits z[t][e] = sum_h x[t][h] * W[e][h], h ascending, in double. */
int orc_logits(const orc_desc* d, const float* w_router, const void* x, int32_t n_tokens,
               double* z) {
  if (!desc_ok(d)) return ORC_EINVAL;
  const int64_t H = d->hidden, E = d->n_experts;
#pragma omp parallel for schedule(static)
  for (int64_t te = 0; te < (int64_t)n_tokens * E; ++te) {
    int64_t t = te / E, e = te % E;
    double acc = 0.0;
    for (int64_t h = 0; h < H; ++h)
      acc += x_at(x, d->act_bf16, t * H + h) * (double)w_router[e * H + h];
    z[te] = acc;
  }
  return ORC_OK;
}

/* a beats b: larger value, or equal value and lower index. */
static int beats(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

/* Index of the best entry among those with allowed[i] != 0, or -1. */
static int argbest(const double* v, const unsigned char* allowed, int n) {
  int best = -1;
  for (int i = 0; i < n; ++i) {
    if (!allowed[i]) continue;
    if (best < 0 || beats(v[i], i, v[best], best)) best = i;
  }
  return best;
}

/* Selection for one token.
 * Sigmoid noaux_tc ("colibri" README, "What's implemented"; DeepSeek-V3-style
 * router): s = sigmoid(z); the correction bias is added for selection only,
 * c = s + bias; experts form n_group contiguous groups; a group's score is the
 * sum of its two largest c; the topk_group best groups are kept; the top_k
 * best c among the kept groups' experts are chosen; their weights are
 * s / sum(s) over the chosen, times routed_scaling.
 * Softmax top-k (the Granite MoE layer of the "Glacial" page): the top_k
 * largest logits are chosen and their weights are the softmax over those k.
 * Ties go to the lowest index everywhere; output is in rank order.
 * Adaptive expert top-p ("colibri" README, "Quick start" knobs: --topp; the
 * pages give the knob and its effect, fewer experts read, not the rule; ours
 * is the nucleus rule over the chosen experts): with 0 < top_p < 1, only the
 * shortest rank prefix whose routing mass reaches top_p of the total is kept
 * -- slot j stays when the mass of the slots before it is below top_p times
 * the total, so at least one -- and the kept weights are renormalized over
 * the prefix; dropped slots get index -1 and weight 0.  Masses are the
 * sigmoid values (or softmax numerators), summed in rank order in double. */
static void select_one(const orc_desc* d, const double* z, const float* bias, int32_t* idx,
                       float* w, double* w64) {
  const int E = d->n_experts, K = d->top_k;
  double* s = (double*)malloc(sizeof(double) * (size_t)E);
  double* c = (double*)malloc(sizeof(double) * (size_t)E);
  unsigned char* cand = (unsigned char*)malloc((size_t)E);
  double wsum = 0.0;
  double* wk = (double*)malloc(sizeof(double) * (size_t)K);

  if (d->router == ORC_ROUTER_SOFTMAX_TOPK) {
    for (int e = 0; e < E; ++e) cand[e] = 1;
    for (int j = 0; j < K; ++j) {
      int b = argbest(z, cand, E);
      idx[j] = b;
      cand[b] = 0;
    }
    double z0 = z[idx[0]];
    for (int j = 0; j < K; ++j) {
      wk[j] = exp(z[idx[j]] - z0);
      wsum += wk[j];
    }
  } else {
    const int G = d->n_group, per = E / G;
    for (int e = 0; e < E; ++e) {
      s[e] = 1.0 / (1.0 + exp(-z[e]));
      c[e] = s[e] + (bias ? (double)bias[e] : 0.0);
    }
    double* gscore = (double*)malloc(sizeof(double) * (size_t)G);
    unsigned char* gallow = (unsigned char*)malloc((size_t)G);
    for (int g = 0; g < G; ++g) {
      /* the two largest c of the group (one value if the group has one expert) */
      int a = -1, b = -1;
      for (int e = g * per; e < (g + 1) * per; ++e) {
        if (a < 0 || beats(c[e], e, c[a], a)) {
          b = a;
          a = e;
        } else if (b < 0 || beats(c[e], e, c[b], b)) {
          b = e;
        }
      }
      gscore[g] = (b < 0) ? c[a] : c[a] + c[b];
      gallow[g] = 1;
    }
    for (int e = 0; e < E; ++e) cand[e] = 0;
    for (int j = 0; j < d->topk_group; ++j) {
      int g = argbest(gscore, gallow, G);
      gallow[g] = 0;
      for (int e = g * per; e < (g + 1) * per; ++e) cand[e] = 1;
    }
    for (int j = 0; j < K; ++j) {
      int b = argbest(c, cand, E);
      idx[j] = b;
      cand[b] = 0;
    }
    for (int j = 0; j < K; ++j) {
      wk[j] = s[idx[j]];
      wsum += wk[j];
    }
    free(gscore);
    free(gallow);
  }
  /* wk[j]: the routing mass of rank j; wsum: their sum in rank order */
  int keep = K;
  if (d->top_p > 0.0 && d->top_p < 1.0) {
    const double thr = d->top_p * wsum;
    double before = 0.0;
    keep = 0;
    while (keep < K && before < thr) before += wk[keep++];
    wsum = before;
  }
  for (int j = 0; j < K; ++j) {
    if (j < keep) {
      wk[j] = wk[j] / wsum * d->routed_scaling;
    } else {
      idx[j] = -1;
      wk[j] = 0.0;
    }
  }
  for (int j = 0; j < K; ++j) {
    if (w) w[j] = (float)wk[j];
    if (w64) w64[j] = wk[j];
  }
  free(s);
  free(c);
  free(cand);
  free(wk);
}

int orc_select(const orc_desc* d, const double* z, const float* bias, int32_t n_tokens,
               int32_t* topk_idx, float* topk_w, double* topk_w64) {
  if (!desc_ok(d)) return ORC_EINVAL;
  const int E = d->n_experts, K = d->top_k;
#pragma omp parallel for schedule(static)
  for (int t = 0; t < n_tokens; ++t)
    select_one(d, z + (int64_t)t * E, bias, topk_idx + (int64_t)t * K,
               topk_w ? topk_w + (int64_t)t * K : NULL,
               topk_w64 ? topk_w64 + (int64_t)t * K : NULL);
  return ORC_OK;
}

int orc_route(const orc_desc* d, const float* w_router, const float* bias, const void* x,
              int32_t n_tokens, int32_t* topk_idx, float* topk_w, double* topk_w64) {
  if (!desc_ok(d)) return ORC_EINVAL;
  if (n_tokens == 0) return ORC_OK;
  double* z = (double*)malloc(sizeof(double) * (size_t)n_tokens * (size_t)d->n_experts);
  int rc = orc_logits(d, w_router, x, n_tokens, z);
  if (rc == ORC_OK) rc = orc_select(d, z, bias, n_tokens, topk_idx, topk_w, topk_w64);
  free(z);
  return rc;
}

/* -------------------------------------------------------------- buckets -- */

/* Batch-union grouping ("colibri" README, "What's implemented": each unique
 * expert of the batch is read once and applied to every position routed to
 * it): a stable counting sort of the flat slots f = t*top_k + j by expert.
 * Slots dropped by adaptive top-p (index -1) are not grouped; their inverse is
 * -1. */
int orc_bucket(int32_t n_tokens, int32_t top_k, int32_t n_experts, const int32_t* topk_idx,
               int32_t* counts, int32_t* offsets, int32_t* entries, int32_t* inverse,
               int32_t* active, int32_t* n_active) {
  const int64_t F = (int64_t)n_tokens * top_k;
  for (int e = 0; e < n_experts; ++e) counts[e] = 0;
  for (int64_t f = 0; f < F; ++f) {
    int e = topk_idx[f];
    if (e == -1) continue;
    if (e < 0 || e >= n_experts) return ORC_EINVAL;
    counts[e] += 1;
  }
  offsets[0] = 0;
  for (int e = 0; e < n_experts; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_experts);
  for (int e = 0; e < n_experts; ++e) fill[e] = offsets[e];
  for (int64_t f = 0; f < F; ++f) {
    int e = topk_idx[f];
    if (e == -1) {
      inverse[f] = -1;
      continue;
    }
    entries[fill[e]] = (int32_t)f;
    inverse[f] = fill[e];
    fill[e] += 1;
  }
  free(fill);
  int na = 0;
  for (int e = 0; e < n_experts; ++e)
    if (counts[e] > 0) active[na++] = e;
  *n_active = na;
  return ORC_OK;
}

/* ----------------------------------------------------------- expert FFN -- */

/* First half of a SwiGLU expert ("iliria" README, "What's implemented":
 * routed-expert SwiGLU, gate and up over one activation): g_r and u_r are the
 * gate and up rows applied to xv[H]; h_r = silu(g_r) * u_r with silu(v) =
 * v / (1 + exp(-v)), in fp64, not rounded.
 * With ebuf (a test tolerance, not part of the layer), also the scale of the
 * error that rounding the terms of g and u makes in h, to first order:
 * e_r = |silu'(g) u| * sum_c |w_gc x_c| + |silu(g)| * sum_c |w_uc x_c|, with
 * silu'(v) = s (1 + v (1 - s)), s = 1 / (1 + exp(-v)). */
static void swiglu_rows(int32_t dtype, const void* gu, const float* gus, int64_t H, int64_t I,
                        const double* xv, double* hbuf, double* ebuf) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < I; ++r) {
    double g = 0.0, u = 0.0;
    for (int64_t c = 0; c < H; ++c) g += weight_at(dtype, gu, gus, H, r, c) * xv[c];
    for (int64_t c = 0; c < H; ++c) u += weight_at(dtype, gu, gus, H, I + r, c) * xv[c];
    double h = g / (1.0 + exp(-g)) * u;
    hbuf[r] = h;
    if (ebuf) {
      double ag = 0.0, au = 0.0;
      for (int64_t c = 0; c < H; ++c) ag += fabs(weight_at(dtype, gu, gus, H, r, c) * xv[c]);
      for (int64_t c = 0; c < H; ++c) au += fabs(weight_at(dtype, gu, gus, H, I + r, c) * xv[c]);
      const double sg = 1.0 / (1.0 + exp(-g));
      const double dsilu = sg * (1.0 + g * (1.0 - sg));
      ebuf[r] = fabs(dsilu * u) * ag + fabs(g * sg) * au;
    }
  }
}

/* SwiGLU expert on one activation vector xv[H] -> y[H]: h from swiglu_rows;
 * when activations are bf16, h is rounded to float and then to bf16 (round to
 * nearest even) before the down projection; y_o = sum_r down[o][r] * h_r. */
static void ffn_one(int32_t dtype, int act_bf16, const void* gu, const float* gus, const void* dn,
                    const float* dns, int64_t H, int64_t I, const double* xv, double* hbuf,
                    double* y) {
  swiglu_rows(dtype, gu, gus, H, I, xv, hbuf, NULL);
  if (act_bf16)
    for (int64_t r = 0; r < I; ++r) hbuf[r] = bf16_to_double(float_to_bf16((float)hbuf[r]));
#pragma omp parallel for schedule(static)
  for (int64_t o = 0; o < H; ++o) {
    double acc = 0.0;
    for (int64_t r = 0; r < I; ++r) acc += weight_at(dtype, dn, dns, I, o, r) * hbuf[r];
    y[o] = acc;
  }
}

static int set_has(const orc_expert_set* set, int32_t e) {
  if (!set || !set->gate_up || !set->down || !set->gate_up[e] || !set->down[e]) return 0;
  if (set->dtype != ORC_BF16) {
    if (!set->gate_up_scale || !set->down_scale) return 0;
    if (!set->gate_up_scale[e] || !set->down_scale[e]) return 0;
  }
  return 1;
}

static int ffn_token(const orc_desc* d, const orc_expert_set* set, int32_t e, int64_t I,
                     const void* x, int64_t t, double* xv, double* hbuf, double* y) {
  if (!set_has(set, e)) return ORC_EMISSING;
  const int64_t H = d->hidden;
  for (int64_t c = 0; c < H; ++c) xv[c] = x_at(x, d->act_bf16, t * H + c);
  ffn_one(set->dtype, d->act_bf16, set->gate_up[e], set->gate_up_scale ? set->gate_up_scale[e] : 0,
          set->down[e], set->down_scale ? set->down_scale[e] : 0, H, I, xv, hbuf, y);
  return ORC_OK;
}

/* The SwiGLU output h (fp64, before any rounding) of one expert over a list
 * of rows, as orc_expert_ffn evaluates it: h[i][r] for token rows[i] / row_div
 * (rows NULL: token i); inter is the expert's intermediate size.  e
 * (nullable) receives the error scale of each h (swiglu_rows). */
int orc_expert_h(const orc_desc* d, const orc_expert_set* set, int32_t expert, int32_t inter,
                 const void* x, const int32_t* rows, int32_t n_rows, int32_t row_div,
                 double* h, double* e) {
  if (!d || d->hidden <= 0 || inter <= 0 || row_div <= 0) return ORC_EINVAL;
  if (!set_has(set, expert)) return ORC_EMISSING;
  const int64_t H = d->hidden;
  double* xv = (double*)malloc(sizeof(double) * (size_t)H);
  for (int32_t i = 0; i < n_rows; ++i) {
    const int64_t t = rows ? rows[i] / row_div : i;
    for (int64_t c = 0; c < H; ++c) xv[c] = x_at(x, d->act_bf16, t * H + c);
    swiglu_rows(set->dtype, set->gate_up[expert],
                set->gate_up_scale ? set->gate_up_scale[expert] : 0, H, inter, xv,
                h + (int64_t)i * inter, e ? e + (int64_t)i * inter : NULL);
  }
  free(xv);
  return ORC_OK;
}

/* One expert over a list of rows: token = rows[i] / row_div (rows NULL: all
 * n_rows tokens in order).  inter is the expert's intermediate size. */
int orc_expert_ffn(const orc_desc* d, const orc_expert_set* set, int32_t expert, int32_t inter,
                   const void* x, const int32_t* rows, int32_t n_rows, int32_t row_div,
                   double* y) {
  if (!d || d->hidden <= 0 || inter <= 0 || row_div <= 0) return ORC_EINVAL;
  const int64_t H = d->hidden;
  double* xv = (double*)malloc(sizeof(double) * (size_t)H);
  double* hb = (double*)malloc(sizeof(double) * (size_t)inter);
  int rc = ORC_OK;
  for (int32_t i = 0; i < n_rows && rc == ORC_OK; ++i) {
    int64_t t = rows ? rows[i] / row_div : i;
    rc = ffn_token(d, set, expert, inter, x, t, xv, hb, y + (int64_t)i * H);
  }
  free(xv);
  free(hb);
  return rc;
}

/* ------------------------------------------------------- bf16 twin band -- */

/* Rounding h to bf16 (act bf16) is a decision that floating point takes: a
 * kernel that accumulates in fp32 in another order lands a value lying very
 * near a rounding midpoint on either side of it, and both roundings are
 * correct results of the layer as defined ("muse-glimmer-intel-serve"
 * introduction: the low-precision twin defines the deviation band).  An h is
 * ambiguous when its float value lies within window * e of the midpoint
 * between its two bf16 neighbours, e being the scale of the error that
 * rounding the terms of its sums makes in h (swiglu_rows); window is then a
 * multiple of the unit roundoff that covers a kernel's accumulation error.
 * For every ambiguous h the other neighbour is also valid; the band of an
 * output is the largest change such alternatives can make to it:
 *   band[t][o] = sum_j |w_tj| * sum_{r ambiguous} |down_o,r| * |h_alt - h_bf16|
 * plus the same sum over the shared expert (weight 1).  Zero when
 * activations are f32. */
static void ffn_band_one(int32_t dtype, const void* gu, const float* gus, const void* dn,
                         const float* dns, int64_t H, int64_t I, const double* xv,
                         double window, double weight, double* dh, double* eb, double* band) {
  swiglu_rows(dtype, gu, gus, H, I, xv, dh, eb);
  for (int64_t r = 0; r < I; ++r) {
    const float hf = (float)dh[r];
    uint32_t bits;
    memcpy(&bits, &hf, 4);
    dh[r] = 0.0;
    if ((bits & 0x7F800000u) == 0x7F800000u) continue;
    const uint32_t lo_bits = bits & 0xFFFF0000u, hi_bits = lo_bits + 0x10000u;
    float lo, hi;
    memcpy(&lo, &lo_bits, 4);
    memcpy(&hi, &hi_bits, 4);
    const double mid = 0.5 * ((double)lo + (double)hi);
    if (fabs((double)hf - mid) <= window * eb[r]) dh[r] = fabs((double)hi - (double)lo);
  }
#pragma omp parallel for schedule(static)
  for (int64_t o = 0; o < H; ++o) {
    double acc = 0.0;
    for (int64_t r = 0; r < I; ++r)
      if (dh[r] != 0.0) acc += fabs(weight_at(dtype, dn, dns, I, o, r)) * dh[r];
    band[o] += weight * acc;
  }
}

int orc_layer_band(const orc_desc* d, const float* w_router, const float* bias,
                   const orc_expert_set* routed, const orc_expert_set* shared, const void* x,
                   int32_t n_tokens, double window, double* band) {
  if (!desc_ok(d) || !(window >= 0.0)) return ORC_EINVAL;
  const int64_t H = d->hidden, K = d->top_k;
  for (int64_t i = 0; i < (int64_t)n_tokens * H; ++i) band[i] = 0.0;
  if (n_tokens == 0 || !d->act_bf16) return ORC_OK;
  const int64_t Is = (int64_t)d->inter * (d->n_shared > 1 ? d->n_shared : 1);
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_tokens * (size_t)K);
  double* w64 = (double*)malloc(sizeof(double) * (size_t)n_tokens * (size_t)K);
  double* xv = (double*)malloc(sizeof(double) * (size_t)H);
  double* dh = (double*)malloc(sizeof(double) * (size_t)Is);
  double* eb = (double*)malloc(sizeof(double) * (size_t)Is);
  int rc = orc_route(d, w_router, bias, x, n_tokens, idx, NULL, w64);
  for (int64_t t = 0; t < n_tokens && rc == ORC_OK; ++t) {
    for (int64_t c = 0; c < H; ++c) xv[c] = x_at(x, 1, t * H + c);
    for (int64_t j = 0; j < K && rc == ORC_OK; ++j) {
      const int32_t e = idx[t * K + j];
      if (e < 0) continue;   /* dropped by adaptive top-p */
      if (!set_has(routed, e)) {
        rc = ORC_EMISSING;
        break;
      }
      ffn_band_one(routed->dtype, routed->gate_up[e],
                   routed->gate_up_scale ? routed->gate_up_scale[e] : 0, routed->down[e],
                   routed->down_scale ? routed->down_scale[e] : 0, H, d->inter, xv, window,
                   fabs(w64[t * K + j]), dh, eb, band + t * H);
    }
    if (rc == ORC_OK && d->n_shared > 0) {
      if (!set_has(shared, 0)) {
        rc = ORC_EMISSING;
        break;
      }
      ffn_band_one(shared->dtype, shared->gate_up[0],
                   shared->gate_up_scale ? shared->gate_up_scale[0] : 0, shared->down[0],
                   shared->down_scale ? shared->down_scale[0] : 0, H, Is, xv, window, 1.0,
                   dh, eb, band + t * H);
    }
  }
  free(idx);
  free(w64);
  free(xv);
  free(dh);
  free(eb);
  return rc;
}

/* ---------------------------------------------------------------- layer -- */

/* The layer's plain definition, token by token: out[t] = sum_j w[t][j] *
 * FFN_{e_tj}(x[t]) (j ascending) + shared(x[t]), in double.  The shared expert
 * is unscaled ("colibri" README, "The idea" and "What's implemented"). */
int orc_layer_forward_per_token(const orc_desc* d, const float* w_router, const float* bias,
                                const orc_expert_set* routed, const orc_expert_set* shared,
                                const void* x, int32_t n_tokens, double* out) {
  if (!desc_ok(d)) return ORC_EINVAL;
  if (n_tokens == 0) return ORC_OK;
  const int64_t H = d->hidden, K = d->top_k;
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_tokens * (size_t)K);
  double* w64 = (double*)malloc(sizeof(double) * (size_t)n_tokens * (size_t)K);
  double* xv = (double*)malloc(sizeof(double) * (size_t)H);
  double* hb = (double*)malloc(sizeof(double) * (size_t)d->inter * (size_t)(d->n_shared > 1 ? d->n_shared : 1));
  double* yj = (double*)malloc(sizeof(double) * (size_t)H);
  double* acc = (double*)malloc(sizeof(double) * (size_t)H);
  int rc = orc_route(d, w_router, bias, x, n_tokens, idx, NULL, w64);
  for (int64_t t = 0; t < n_tokens && rc == ORC_OK; ++t) {
    for (int64_t o = 0; o < H; ++o) acc[o] = 0.0;
    for (int64_t j = 0; j < K && rc == ORC_OK; ++j) {
      if (idx[t * K + j] < 0) continue;   /* dropped by adaptive top-p */
      rc = ffn_token(d, routed, idx[t * K + j], d->inter, x, t, xv, hb, yj);
      for (int64_t o = 0; o < H; ++o) acc[o] += w64[t * K + j] * yj[o];
    }
    if (rc == ORC_OK && d->n_shared > 0) {
      rc = ffn_token(d, shared, 0, (int64_t)d->inter * d->n_shared, x, t, xv, hb, yj);
      for (int64_t o = 0; o < H; ++o) acc[o] += yj[o];
    }
    for (int64_t o = 0; o < H; ++o) out[t * H + o] = acc[o];
  }
  free(idx);
  free(w64);
  free(xv);
  free(hb);
  free(yj);
  free(acc);
  return rc;
}

/* The same layer evaluated the batch-union way: route every token, bucket the
 * slots by expert, apply each active expert once to all of its slots, then
 * combine per token in slot order.  Same arithmetic per (token, expert) as the
 * per-token form, so the two agree bit for bit. */
int orc_layer_forward(const orc_desc* d, const float* w_router, const float* bias,
                      const orc_expert_set* routed, const orc_expert_set* shared, const void* x,
                      int32_t n_tokens, double* out, int32_t* topk_idx, float* topk_w) {
  if (!desc_ok(d)) return ORC_EINVAL;
  if (n_tokens == 0) return ORC_OK;
  const int64_t H = d->hidden, K = d->top_k, E = d->n_experts;
  const int64_t F = (int64_t)n_tokens * K;
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)F);
  double* w64 = (double*)malloc(sizeof(double) * (size_t)F);
  int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* entries = (int32_t*)malloc(sizeof(int32_t) * (size_t)F);
  int32_t* inverse = (int32_t*)malloc(sizeof(int32_t) * (size_t)F);
  int32_t* active = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  double* Y = (double*)malloc(sizeof(double) * (size_t)F * (size_t)H);
  double* S = (double*)malloc(sizeof(double) * (size_t)H);
  double* xv = (double*)malloc(sizeof(double) * (size_t)H);
  double* hb = (double*)malloc(sizeof(double) * (size_t)d->inter * (size_t)(d->n_shared > 1 ? d->n_shared : 1));
  int32_t n_active = 0;
  int rc = orc_route(d, w_router, bias, x, n_tokens, idx, topk_w, w64);
  if (rc == ORC_OK)
    rc = orc_bucket(n_tokens, (int32_t)K, (int32_t)E, idx, counts, offsets, entries, inverse,
                    active, &n_active);
  for (int32_t a = 0; a < n_active && rc == ORC_OK; ++a) {
    const int32_t e = active[a];
    for (int32_t p = offsets[e]; p < offsets[e + 1] && rc == ORC_OK; ++p) {
      const int32_t f = entries[p];
      rc = ffn_token(d, routed, e, d->inter, x, f / K, xv, hb, Y + (int64_t)f * H);
    }
  }
  for (int64_t t = 0; t < n_tokens && rc == ORC_OK; ++t) {
    for (int64_t o = 0; o < H; ++o) {
      double acc = 0.0;
      for (int64_t j = 0; j < K; ++j)
        if (idx[t * K + j] >= 0) acc += w64[t * K + j] * Y[(t * K + j) * H + o];
      out[t * H + o] = acc;
    }
    if (d->n_shared > 0) {
      rc = ffn_token(d, shared, 0, (int64_t)d->inter * d->n_shared, x, t, xv, hb, S);
      for (int64_t o = 0; o < H && rc == ORC_OK; ++o) out[t * H + o] += S[o];
    }
  }
  if (topk_idx && rc == ORC_OK) memcpy(topk_idx, idx, sizeof(int32_t) * (size_t)F);
  free(idx);
  free(w64);
  free(counts);
  free(offsets);
  free(entries);
  free(inverse);
  free(active);
  free(Y);
  free(S);
  free(xv);
  free(hb);
  return rc;
}

/* ------------------------------------------------------- requantizer -- */

/* OCP FP8 E4M3 (the "fn" encoding: no infinities, S.1111.111 is NaN): the
 * value of a byte from its sign, 4-bit exponent (bias 7) and 3-bit mantissa;
 * exponent 0 is subnormal, m/8 * 2^-6. */
static double e4m3_value(uint8_t b) {
  const int e = (b >> 3) & 0xF, m = b & 7;
  double v;
  if (e == 15 && m == 7) v = NAN;
  else if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp(8.0 + (double)m, e - 10);
  return (b & 0x80) ? -v : v;
}

int orc_decode_e4m3(const uint8_t* b, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(b[i]);
  return ORC_OK;
}

/* The offline FP8 -> int4 converter ("colibri" README, "What's implemented":
 * FP8 weights with 128x128 block scales are dequantized and requantized to
 * the engine's per-row int4 container).  The pages fix neither the int4 range
 * nor the rounding; our reading: w = e4m3(b) * block scale, exact in double;
 * per row m = max |w|; scale = float(m / 7), nearest even; q = nearest-even
 * of w / scale, clamped to [-7, 7] (q = 0 where the scale is 0); codes packed
 * two per byte, low nibble first.  block_scales: [ceil(rows/block)]
 * [ceil(cols/block)] fp32.  A NaN code is an error (ORC_EINVAL). */
int orc_requant_fp8_int4(const uint8_t* fp8, const float* block_scales, int64_t rows,
                         int64_t cols, int32_t block, uint8_t* codes, float* scales) {
  if (rows < 0 || cols <= 0 || (cols & 1) || block <= 0) return ORC_EINVAL;
  const int64_t bcols = (cols + block - 1) / block;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t r = 0; r < rows; ++r) {
    const uint8_t* in = fp8 + r * cols;
    const float* bs = block_scales + (r / block) * bcols;
    double m = 0.0;
    for (int64_t c = 0; c < cols; ++c) {
      const double w = e4m3_value(in[c]) * (double)bs[c / block];
      if (isnan(w)) bad = 1;
      if (fabs(w) > m) m = fabs(w);
    }
    const float s = (float)(m / 7.0);
    scales[r] = s;
    for (int64_t c = 0; c < cols; c += 2) {
      int q[2];
      for (int k = 0; k < 2; ++k) {
        const double w = e4m3_value(in[c + k]) * (double)bs[(c + k) / block];
        double v = s == 0.0f ? 0.0 : rint(w / (double)s);
        if (v > 7.0) v = 7.0;
        if (v < -7.0) v = -7.0;
        q[k] = (int)v;
      }
      codes[r * (cols / 2) + c / 2] = (uint8_t)(((unsigned)q[0] & 0xFu) | (((unsigned)q[1] & 0xFu) << 4));
    }
  }
  return bad ? ORC_EINVAL : ORC_OK;
}

/* ---------------------------------------------------------------- stack -- */

/* RMSNorm with unit gain: v / sqrt(mean(v^2) + eps), in double, rounded to
 * float.  (Layer glue for stacked MoE layers; the pages fix no norm for the
 * routed path itself.) */
int orc_rmsnorm(const float* x, int32_t n_tokens, int32_t hidden, double eps, float* out) {
  for (int64_t t = 0; t < n_tokens; ++t) {
    double ss = 0.0;
    for (int64_t h = 0; h < hidden; ++h) {
      double v = (double)x[t * hidden + h];
      ss += v * v;
    }
    double den = sqrt(ss / (double)hidden + eps);
    for (int64_t h = 0; h < hidden; ++h) out[t * hidden + h] = (float)((double)x[t * hidden + h] / den);
  }
  return ORC_OK;
}

/* Residual stream update x <- x + float(y): the layer output rounds to float
 * first, then one float addition. */
int orc_residual_add(float* x, const double* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    float yf = (float)y[i];
    x[i] = (float)((double)x[i] + (double)yf);
  }
  return ORC_OK;
}

void orc_set_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int32_t orc_max_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}
