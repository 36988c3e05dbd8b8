/*
 * moe_oracle.h -- plain, slow CPU oracle of the routed MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header or table with the HIP path in quantized_expert_ffn_sigmoid_amd/.
 *
 * Everything is host memory.  Floating point accumulates in double; inputs
 * (f32, bf16, integer codes times f32 scales) widen exactly to double.
 * Parity status of every function is listed in moe_oracle.c's header.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

enum { ORC_BF16 = 1, ORC_I4 = 2, ORC_I2 = 3, ORC_I8 = 4 };
enum { ORC_ROUTER_SIGMOID_NOAUX_TC = 0, ORC_ROUTER_SOFTMAX_TOPK = 1 };
enum { ORC_OK = 0, ORC_EINVAL = 1, ORC_EMISSING = 2 };

typedef struct {
  int32_t hidden, inter, n_experts, top_k;
  int32_t router;             /* ORC_ROUTER_*                                   */
  int32_t n_group, topk_group;
  double routed_scaling;
  int32_t expert_dtype;       /* ORC_BF16 | ORC_I4 | ORC_I2 | ORC_I8            */
  int32_t act_bf16;           /* 1: x is bf16 and h is rounded to bf16          */
  int32_t n_shared;           /* 0 or 1                                         */
  int32_t shared_dtype;       /* ORC_BF16 | ORC_I4 | ORC_I2 | ORC_I8            */
  double top_p;               /* adaptive expert top-p; off unless 0 < p < 1    */
} orc_desc;

/* One expert set.  Each table has one entry per expert; an entry may be NULL
 * when that expert is never evaluated (then evaluating it is ORC_EMISSING).
 * gate_up[e] -> [2I rows][H cols], rows 0..I-1 gate, I..2I-1 up;
 * down[e]    -> [H rows][I cols];  codes packed along the column (input) axis.
 * Scale tables are unused for bf16 weights. */
typedef struct {
  int32_t dtype;
  const void* const* gate_up;
  const float* const* gate_up_scale;
  const void* const* down;
  const float* const* down_scale;
} orc_expert_set;

int orc_decode_codes(int32_t dtype, const uint8_t* packed, int64_t n, int8_t* out);
int orc_dequant_rows(int32_t dtype, const void* codes, const float* scales, int64_t cols,
                     int64_t row0, int64_t n_rows, float* out);
int orc_logits(const orc_desc* d, const float* w_router, const void* x, int32_t n_tokens,
               double* z);
int orc_select(const orc_desc* d, const double* z, const float* bias, int32_t n_tokens,
               int32_t* topk_idx, float* topk_w, double* topk_w64);
int orc_route(const orc_desc* d, const float* w_router, const float* bias, const void* x,
              int32_t n_tokens, int32_t* topk_idx, float* topk_w, double* topk_w64);
int orc_bucket(int32_t n_tokens, int32_t top_k, int32_t n_experts, const int32_t* topk_idx,
               int32_t* counts, int32_t* offsets, int32_t* entries, int32_t* inverse,
               int32_t* active, int32_t* n_active);
int orc_expert_ffn(const orc_desc* d, const orc_expert_set* set, int32_t expert, int32_t inter,
                   const void* x, const int32_t* rows, int32_t n_rows, int32_t row_div,
                   double* y);
/* The expert's SwiGLU output h[n_rows][inter] in fp64 before any rounding
 * (rows as orc_expert_ffn); e (nullable) receives each h's error scale
 * |silu'(g) u| sum|w_g x| + |silu(g)| sum|w_u x| (a test tolerance). */
int orc_expert_h(const orc_desc* d, const orc_expert_set* set, int32_t expert, int32_t inter,
                 const void* x, const int32_t* rows, int32_t n_rows, int32_t row_div,
                 double* h, double* e);
int orc_layer_forward(const orc_desc* d, const float* w_router, const float* bias,
                      const orc_expert_set* routed, const orc_expert_set* shared, const void* x,
                      int32_t n_tokens, double* out, int32_t* topk_idx, float* topk_w);
int orc_layer_forward_per_token(const orc_desc* d, const float* w_router, const float* bias,
                                const orc_expert_set* routed, const orc_expert_set* shared,
                                const void* x, int32_t n_tokens, double* out);
/* Output band of the bf16 rounding of h (act bf16 only; zero otherwise):
 * band[t][o] bounds the change of out[t][o] when every h whose float value
 * lies within window * e of a bf16 rounding midpoint takes the other
 * rounding, e being the first-order scale of the error that rounding the
 * terms of g and u makes in h (orc_expert_h).  A test tolerance, not part of
 * the layer. */
int orc_layer_band(const orc_desc* d, const float* w_router, const float* bias,
                   const orc_expert_set* routed, const orc_expert_set* shared, const void* x,
                   int32_t n_tokens, double window, double* band);
int orc_rmsnorm(const float* x, int32_t n_tokens, int32_t hidden, double eps, float* out);
int orc_residual_add(float* x, const double* y, int64_t n);
void orc_set_threads(int32_t n);
int32_t orc_max_threads(void);

/* FP8 (OCP E4M3, no infinities) decode, and the FP8 -> int4 requantizer. */
int orc_decode_e4m3(const uint8_t* b, int64_t n, double* out);
int orc_requant_fp8_int4(const uint8_t* fp8, const float* block_scales, int64_t rows,
                         int64_t cols, int32_t block, uint8_t* codes, float* scales);

#endif
