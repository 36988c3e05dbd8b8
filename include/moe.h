/*
 * moe.h -- C ABI of the MI355X (gfx950) routed MoE layer forward.
 *
 * The layer (pages: "colibri" README, sections "The idea" and "What's
 * implemented"; "iliria" README, section "What's implemented"):
 *   1. a DeepSeek-V3-style sigmoid router (noaux_tc): sigmoid scores, a
 *      correction bias used for selection only, group-limited top-k, weights
 *      renormalised over the chosen experts and multiplied by
 *      routed_scaling_factor -- or, for Granite-shaped layers ("Glacial" page),
 *      a softmax top-k router;
 *   2. batch-union grouping: every unique expert of the batch is read once and
 *      applied to every position routed to it;
 *   3. SwiGLU experts stored as packed int4 / packed int2 codes with per-row
 *      scales (or bf16), dequantized on use;
 *   4. the weighted combine of the routed experts plus the shared expert.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns all
 *     memory; the library allocates nothing of its own for the data, so it
 *     is safe to call from several host threads on different streams.  Two
 *     exceptions: moe_layer_forward_noalloc runs on a workspace of the
 *     library's own, one per GPU; and layers with a bf16 shared expert, on
 *     batches of 256 tokens or more, run that expert's two dense GEMMs
 *     through hipBLASLt, with a handle per GPU and one algorithm per shape
 *     that the first such call outside graph capture creates and keeps
 *     (a call captured before any has runs the grouped-GEMM tiles instead).
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronise: results are valid once the stream has
 *     reached the enqueued work.  A device-side fault surfaces at the caller's
 *     next synchronisation.
 *   - Arguments are validated on the host before anything is launched; a
 *     rejected call launches nothing.  No C++ exception crosses this ABI.
 *   - Row-major layouts throughout.  Packed codes run along the input axis
 *     of an [out][in] matrix: int4 element i of a row sits in byte i/2, low
 *     nibble first (bits 0-3 = even element), two's complement; int2 element i
 *     sits in byte i/4 at bits 2(i%4)..2(i%4)+1, two's complement.  One fp32
 *     scale per output row ("per-row scales", "colibri" README).
 *   - Ties in every selection go to the lowest index; router outputs are in
 *     rank order (descending score, then ascending expert index).
 *   - Non-finite inputs are outside the contract.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* null/misaligned pointer, inconsistent descriptor      */
  MOE_EUNSUPPORTED = 2,  /* valid but outside what the kernels handle (shapes)    */
  MOE_EWORKSPACE = 3,    /* ws_bytes smaller than moe_workspace_bytes()           */
  MOE_EHIP = 4           /* a HIP launch or runtime call failed                   */
} moe_status;

/* Weight containers ("colibri" README, "What's implemented": packed int4 and
 * packed int2 with per-row scales, validated against an int8 container):
 * MOE_I4: element i of a row in byte i/2, low nibble first, two's complement;
 * MOE_I2: element i in byte i/4 at bits 2(i%4), two's complement; MOE_I8:
 * element i is byte i, two's complement.  Integer weights are code * (fp32
 * row scale).  MOE_BF16: bf16 weights, no scales. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_I4 = 2, MOE_I2 = 3, MOE_I8 = 4 } moe_dtype;

typedef enum { MOE_ROUTER_SIGMOID_NOAUX_TC = 0, MOE_ROUTER_SOFTMAX_TOPK = 1 } moe_router;

/* Layer shape and numerics (plain data, passed by host pointer). */
typedef struct {
  int32_t hidden;          /* H: model width                                          */
  int32_t inter;           /* I: routed expert intermediate size                      */
  int32_t n_experts;       /* E: routed experts (<= 1024)                             */
  int32_t top_k;           /* k: experts per token (<= 32, <= E)                      */
  int32_t router;          /* moe_router                                              */
  int32_t n_group;         /* sigmoid router: contiguous expert groups (1 = none)     */
  int32_t topk_group;      /* sigmoid router: groups kept per token                   */
  float routed_scaling;    /* routed_scaling_factor (1.0 for softmax layers)          */
  int32_t expert_dtype;    /* MOE_I4 | MOE_I2 | MOE_I8 | MOE_BF16                     */
  int32_t act_dtype;       /* MOE_F32 | MOE_BF16: type of x; with MOE_BF16 the        */
                           /* SwiGLU output h is rounded to bf16 before the down     */
                           /* projection                                             */
  int32_t n_shared;        /* 0 or 1 shared expert (intermediate size n_shared * I)   */
  int32_t shared_dtype;    /* MOE_I4 | MOE_I2 | MOE_I8 | MOE_BF16                     */
  float norm_eps;          /* RMSNorm epsilon used by moe_stack_forward               */
  float top_p;             /* adaptive expert top-p ("colibri" README, "Quick start" */
                           /* knob --topp): 0 (or >= 1) = off; 0 < top_p < 1 keeps, */
                           /* per token, the shortest rank prefix of the top_k      */
                           /* whose routing mass reaches top_p of their total (at   */
                           /* least one expert) and renormalizes its weights;       */
                           /* dropped slots get topk_idx -1 and topk_w 0.  Masses:  */
                           /* the sigmoid values (softmax: exp(z - z_max)), summed  */
                           /* in rank order in fp64; slot j stays when the mass     */
                           /* before it is < top_p * total.  NaN or < 0: MOE_EINVAL */
} moe_layer_desc;

/* One expert set: E routed experts, or the n_shared shared expert(s).
 * Expert e's gate/up matrix is [2I rows][H] (rows 0..I-1 gate, I..2I-1 up) at
 * gate_up + e*gate_up_stride bytes; its down matrix is [H rows][I] at
 * down + e*down_stride.  Scales (fp32, one per row) likewise; NULL for bf16.
 * Strides let the caller keep each expert as one contiguous blob (codes and
 * scales side by side) or keep each tensor contiguous across experts.
 * Code and scale rows must be 16-byte aligned. */
typedef struct {
  const void* gate_up;
  int64_t gate_up_stride;
  const float* gate_up_scale;
  int64_t gate_up_scale_stride;
  const void* down;
  int64_t down_stride;
  const float* down_scale;
  int64_t down_scale_stride;
} moe_expert_set;

typedef struct {
  const float* w_router;   /* [E][H] fp32                                   */
  const float* bias;       /* [E] fp32 correction bias, nullable            */
  moe_expert_set routed;   /* E experts of expert_dtype                     */
  moe_expert_set shared;   /* n_shared experts of shared_dtype (if any)     */
} moe_layer_weights;

/* Bytes of workspace moe_layer_forward / moe_stack_forward / moe_route /
 * moe_expert_ffn need for n_tokens tokens (or rows).  Host-only and pure.
 * Returns 0 for an invalid descriptor. */
size_t moe_workspace_bytes(const moe_layer_desc* d, int32_t n_tokens);

/* Router: logits z = x W_r^T accumulated in fp64, then selection.
 * Sigmoid noaux_tc ("colibri" README, "What's implemented"): s = sigmoid(z);
 * c = s + bias; groups are n_group contiguous ranges of E/n_group experts;
 * a group scores the sum of its two largest c; the topk_group best groups are
 * kept; the top_k largest c among their experts are chosen; topk_w[j] =
 * s_j / sum(s over the chosen) * routed_scaling.
 * Softmax top-k (Granite MoE layer, "Glacial" page): the top_k largest z are
 * chosen; topk_w = softmax over the chosen z, times routed_scaling.
 * x: [n_tokens][H] of act_dtype.  Outputs: topk_idx [n_tokens][k] int32,
 * topk_w [n_tokens][k] fp32 (with top_p, dropped slots: -1 and 0).  Errors:
 * MOE_EINVAL (bad descriptor or pointer), MOE_EWORKSPACE. */
moe_status moe_route(const moe_layer_desc* d, const float* w_router, const float* bias,
                     const void* x, int32_t n_tokens, int32_t* topk_idx, float* topk_w,
                     void* ws, size_t ws_bytes, void* stream);

/* Batch-union grouping ("colibri" README, "What's implemented"): a stable
 * counting sort of the flat slots f = t*top_k + j by expert.
 *   counts[E]    slots per expert;  offsets[E+1] exclusive prefix sum;
 *   entries[F]   the slots f, sorted by (expert, f);  inverse[F]: inverse[entries[p]] = p;
 *   active[E]    experts with counts > 0, ascending (first n_active entries valid);
 *   n_active[1]  their number.  F = n_tokens * top_k.
 * Index -1 marks a slot dropped by adaptive top-p: it is left out of every
 * output and its inverse is -1.  Other indices outside [0, E) are a caller
 * error (not detectable on the host: such slots are treated the same way).
 * ws/ws_bytes are unused (pass NULL/0). */
moe_status moe_bucket(int32_t n_tokens, int32_t top_k, int32_t n_experts, const int32_t* topk_idx,
                      int32_t* counts, int32_t* offsets, int32_t* entries, int32_t* inverse,
                      int32_t* active, int32_t* n_active, void* ws, size_t ws_bytes, void* stream);

/* One expert (dequant-on-use SwiGLU; "iliria" README, "What's implemented")
 * on a list of activation rows: y[i] = down(silu(gate x_t) * up x_t) with
 * t = rows[i] / row_div (rows NULL: t = i).  shared = 0 selects routed expert
 * `expert` of `set` (dtype expert_dtype, intermediate I); shared = 1 the shared
 * expert (shared_dtype, intermediate n_shared*I; `expert` must be 0).
 * x: [*][H] act_dtype; y: [n_rows][H] fp32.  Workspace: moe_workspace_bytes(d,
 * n_rows).  Runs on the GEMV kernels: MOE_EUNSUPPORTED when they do not cover
 * the expert's shapes. */
moe_status moe_expert_ffn(const moe_layer_desc* d, const moe_expert_set* set, int32_t shared,
                          int32_t expert, const void* x, const int32_t* rows, int32_t n_rows,
                          int32_t row_div, float* y, void* ws, size_t ws_bytes, void* stream);

/* The whole routed layer ("colibri" README, "The idea" -- a shared expert
 * beside the routed ones -- and "What's implemented" -- the sigmoid router,
 * batch-union grouping and the routed_scaling-weighted combine; "iliria"
 * README, "What's implemented": the SwiGLU expert over one activation): route,
 * bucket, apply each active expert once to all of its tokens, and combine:
 * out[t] = sum_j topk_w[t][j] * FFN_{e_tj}(x_t) (j ascending) + shared(x_t).  x: [n_tokens][H] act_dtype; out: [n_tokens][H]
 * fp32.  topk_idx_out / topk_w_out ([n_tokens][k]) are optional copies of the
 * routing.  Workspace: moe_workspace_bytes(d, n_tokens).
 * Two expert paths: up to 16 tokens, dequant-on-use GEMV kernels; more
 * tokens with act_dtype MOE_BF16, int4 or bf16 experts, H a multiple of 256
 * and I (and n_shared*I) multiples of 128, a grouped GEMM on the matrix cores
 * over 64-row bucket tiles (else the GEMV kernels).  A descriptor is valid
 * when one path covers it; a call whose batch size selects a path that does
 * not returns MOE_EUNSUPPORTED. */
moe_status moe_layer_forward(const moe_layer_desc* d, const moe_layer_weights* w, const void* x,
                             int32_t n_tokens, float* out, int32_t* topk_idx_out,
                             float* topk_w_out, void* ws, size_t ws_bytes, void* stream);

/* Stage timing hook for moe_layer_forward_ex: when non-NULL, `events` is a
 * (host) array of 2*MOE_N_STAGES hipEvent_t handles (entries may be NULL);
 * events[2s] is recorded on `stream` right before the launches of stage s and
 * events[2s+1] right after them.  While the stream is being captured into a
 * graph the records are external event nodes, so each replay times the stage. */
/* Decode batches (<= 16 tokens) whose shared expert streams through the
 * GEMV ring (sigmoid router, <= 256 experts) run the shared expert's gate/up
 * inside the ROUTE stage (the logits launch holds it).  With 2..16 tokens the
 * selection launch, also in ROUTE, holds its down projection; GATE_UP and
 * DOWN then hold the routed experts only.  With one token (int4, int8 or
 * bf16 experts on the ring): ROUTE holds the logits and the shared gate/up;
 * GATE_UP holds the selection and grouping (run inside every routed gate/up
 * block) and the routed gate/up; DOWN holds the routed and shared down
 * projections and the combine in one launch; BUCKET and COMBINE are empty. */
enum {
  MOE_STAGE_ROUTE = 0,     /* router logits + selection (+ grouping, for <= 16 tokens) */
  MOE_STAGE_BUCKET = 1,    /* batch-union grouping (empty when fused into ROUTE)      */
  MOE_STAGE_GATE_UP = 2,   /* gate/up + SwiGLU of the routed (and shared) experts    */
  MOE_STAGE_DOWN = 3,      /* down projections of the routed (and shared) experts    */
  MOE_STAGE_COMBINE = 4,   /* weighted combine (+ residual in stacks)                 */
  MOE_N_STAGES = 5
};
typedef struct {
  void* const* events;     /* (host) [2*MOE_N_STAGES] hipEvent_t, nullable */
  float* h_f32;            /* test hook, nullable: receives the SwiGLU output h  */
                           /* of every routed row before any bf16 rounding,      */
                           /* fp32 [n_tokens*top_k][I] by bucket position (rows  */
                           /* past the grouped slots untouched), then the shared */
                           /* expert's [n_tokens][n_shared*I]                    */
} moe_launch_opts;

moe_status moe_layer_forward_ex(const moe_layer_desc* d, const moe_layer_weights* w,
                                const void* x, int32_t n_tokens, float* out,
                                int32_t* topk_idx_out, float* topk_w_out, void* ws,
                                size_t ws_bytes, void* stream, const moe_launch_opts* opts);

/* Stack glue.  The pages describe one MoE layer; the stacked workloads (a
 * 24-layer Granite-shaped stack and 8 stacked GLM-shaped layers) need the
 * residual and the pre-norm between layers, which the pages leave to the
 * surrounding model.  moe_rmsnorm and moe_stack_forward provide that glue
 * with the plainest reading: RMSNorm with unit gain (eps from the descriptor,
 * 1e-6 in those stacks), residual added in fp32.
 *
 * RMSNorm with unit gain, out = x / sqrt(mean(x^2) + eps), computed in fp64
 * and rounded to fp32.  x, out: [n_tokens][hidden] fp32 (may alias). */
moe_status moe_rmsnorm(const float* x, int32_t n_tokens, int32_t hidden, float eps, float* out,
                       void* stream);

/* A pre-norm residual stack of n_layers MoE layers of one shape:
 * for each layer l: y_l = MoE_l(RMSNorm(x)); x = x + y_l.
 * layers: (host) array of n_layers weight sets; x: [n_tokens][H] fp32, input
 * of layer 0 on entry and the final residual stream on return (act_dtype
 * must be MOE_F32).  y_layers: optional [n_layers][n_tokens][H] fp32 copy of
 * every layer's MoE output.  Workspace: moe_workspace_bytes(d, n_tokens). */
moe_status moe_stack_forward(const moe_layer_desc* d, const moe_layer_weights* layers,
                             int32_t n_layers, float* x, int32_t n_tokens, float* y_layers,
                             void* ws, size_t ws_bytes, void* stream);

/* Test hook: dequantized weights of rows [row0, row0+n_rows) of one [rows][cols]
 * matrix.  out_f32[r][c] = float(q) * scale[row], one fp32 multiply rounded to
 * nearest even (for bf16 weights: the widened value).  out_bf16_codes
 * (nullable, int formats only) receives bf16(q), exact for |q| <= 8. */
moe_status moe_dequant_rows(int32_t dtype, const void* codes, const float* scales, int32_t cols,
                            int32_t row0, int32_t n_rows, float* out_f32,
                            uint16_t* out_bf16_codes, void* stream);

/* FP8 -> int4 requantizer: the step that builds the MOE_I4 container from an
 * FP8 checkpoint ("colibri" README, "What's implemented": the offline
 * converter dequantizes 128x128 block scales and requantizes to the engine's
 * container).  fp8: [rows][cols] OCP E4M3 bytes (no NaN codes; a NaN code
 * gives an unspecified result for its row), 8-byte aligned; block_scales:
 * [ceil(rows/block)][ceil(cols/block)] fp32; w = e4m3 * block scale (exact).
 * Per row: scales[r] = float(m / 7) for m = max |w| (nearest even); codes
 * [rows][cols/2] (4-byte aligned) = nearest-even(w / scales[r]) clamped to
 * [-7, 7] (0 where the scale is 0), low nibble first.  cols a multiple of 8,
 * at most 8192; block a multiple of 8 (else MOE_EUNSUPPORTED).  Matrices
 * stacked along rows share one call when rows per matrix is a multiple of
 * block. */
moe_status moe_requant_fp8_int4(const uint8_t* fp8, const float* block_scales, int32_t rows,
                                int32_t cols, int32_t block, uint8_t* codes, float* scales,
                                void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): moe_layer_forward
 * on a workspace the library carries itself, so the caller passes only
 * inputs and outputs.  The workspace is a device array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes per GPU (one copy on each GPU the library
 * runs on, held until the process ends), taken on the device that `stream`
 * runs on.  The call allocates nothing and runs the same kernels, with the
 * same results, as moe_layer_forward.  Every call on one GPU uses that GPU's
 * array: calls that overlap on one GPU (several streams or host threads)
 * race and give undefined results; calls ordered on one stream are safe.  The
 * array keeps the last call's contents; no kernel relies on its initial
 * contents.  Errors: those of moe_layer_forward, and MOE_EWORKSPACE (nothing
 * launched) when moe_workspace_bytes(d, n_tokens) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES (GLM-scale layers, H 6144 and I 2048: up to 40
 * tokens). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
moe_status moe_layer_forward_noalloc(const moe_layer_desc* d, const moe_layer_weights* w,
                                     const void* x, int32_t n_tokens, float* out,
                                     int32_t* topk_idx_out, float* topk_w_out, void* stream);

const char* moe_status_str(moe_status s);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
