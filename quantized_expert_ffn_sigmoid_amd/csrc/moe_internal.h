// moe_internal.h -- device helpers and the launch interface between the C ABI
// (moe_capi.cpp) and the gfx950 kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kDecodeTokens = 16;   // router logits GEMV path handles up to this many tokens
// Size of the workspace moe_layer_forward_noalloc carries per GPU.
constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;

// ------------------------------------------------------------ device helpers

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// ---------------------------------------------------------- launch structs

// Device view of one expert set; all strides in bytes.
struct ExpertSetDev {
  const uint8_t* gu;
  int64_t gu_stride;
  const uint8_t* gus;
  int64_t gus_stride;
  const uint8_t* dn;
  int64_t dn_stride;
  const uint8_t* dns;
  int64_t dns_stride;
};

// Per-slot records written by the decode grouping, so that an expert GEMV
// block learns its whole assignment from one 32-byte read instead of a chain
// of dependent lookups.  slot_tab[s * kSlotRec + ...] for active slot s <
// n_tab: {expert, first bucket position, rows, flat slot of row 0, flat slot
// of row 1 (or -1)}; expert -1 for s >= n_active.  pos_e[p]: the expert of
// bucket position p, or -1 for positions past the grouped slots.
constexpr int kSlotRec = 8;
struct SlotTables {
  int32_t* slot_tab = nullptr;
  int32_t n_tab = 0;
  int32_t* pos_e = nullptr;
};

// How a GEMV block finds its expert and rows.
//  routed: block slot -> expert active[slot] (slots >= n_active exit);
//          bucket positions p in [offsets[e], offsets[e+1]); slot f = entries[p];
//          token = f / top_k.
//  list:   expert = fixed_expert; i in [0, n_rows); token = rows ? rows[i]/row_div : i.
struct RowSource {
  int routed;
  const int32_t* active;
  const int32_t* n_active;
  const int32_t* offsets;
  const int32_t* entries;
  const int32_t* slot_tab;   // optional (SlotTables), n_slots records
  const int32_t* pos_e;      // optional (SlotTables)
  int32_t top_k;
  int32_t fixed_expert;
  const int32_t* rows;
  int32_t n_rows;
  int32_t row_div;
};

// GEMV geometry of one matrix for an input length K: a unit is kc K-chunks
// of lpr lanes per row, rpp rows per unit (lpr * rpp = 64).
struct MatGeo {
  int32_t kc, lpr, rpp;
};

// Sliced copies of activation rows for up to two weight formats (epg 0 or
// dst null: skipped); see GemvArgs for the layout.
struct SliceReq {
  int32_t epg_a, epg_b;
  void* dst_a;
  void* dst_b;
};

// Router selection parameters (one layer).
struct SelectParams {
  int32_t E, K, G, topk_group, softmax;
  float scaling;
  double top_p;   // adaptive expert top-p, active when 0 < top_p < 1
  // nullable (sigmoid router): [T][E][2] the score s = sigmoid(z) and the
  // biased score s + bias of every expert, written by the logits launch
  // (the same fp64 operations the selection would run)
  const double* zsc;
};

// Routing work that runs in the leading blocks of a shared-expert GEMV launch
// (decode): the router logits (one block per expert) in the gate/up launch,
// the selection and grouping (one block) in the down launch.  The shared
// expert does not depend on the routing, so its weights stream while the
// router's latency-bound steps run.
struct PreArgs {
  int32_t kind;     // kPreLogits or kPreSelect
  int32_t blocks;   // leading blocks of the launch that run it
  // router logits
  const float* w_router;
  const void* x;
  int32_t act_bf16, T, H, E;
  double* z;
  SliceReq sr;
  double* zsc;          // nullable: also write the scores (SelectParams::zsc)
  const float* zbias;   // the router bias for them (nullable)
  // selection + grouping
  SelectParams sp;
  const double* zin;
  const float* bias;
  int32_t* idx;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* entries;
  int32_t* inverse;
  int32_t* active;
  int32_t* n_active;
  SlotTables tb;
  // one-token gate/up launch only: the shared expert's down projection (bf16
  // weights [H][Is], Is = kSdnIs), run by the waves that do not select; null
  // when the down launch computes it
  const uint8_t* sdn;
  const void* sdn_h;    // the shared h, sliced for that matrix
  float* sdn_out;       // [H] the shared expert's output
  int32_t sdn_rpb;      // output rows per block (set by the launch)
};
constexpr int kPreLogits = 1, kPreSelect = 2;
constexpr int kSdnIs = 2048;   // shared intermediate size of that variant

// One GEMV launch: the routed experts of a bucket (or a fixed expert over a
// row list) and, optionally, the shared expert over tokens 0..n_tok-1.
struct GemvArgs {
  ExpertSetDev w;          // routed set (or the set of the fixed expert)
  ExpertSetDev ws;         // shared set
  RowSource src;
  int32_t has_shared, n_tok;
  int32_t H, I, Is;        // Is: shared intermediate size
  int32_t n_slots;         // routed slots in the grid
  const void* x;           // gate/up input rows [*][H] (act dtype)
  const void* x_s;         // gate/up input rows of the shared expert (null: x)
  void* h;                 // routed h rows [bucket position][I] (act dtype)
  void* h_s;               // shared h rows [token][Is]
  // Row layouts.  A "sliced" row of K activations, for a weight format of EPG
  // elements per 16-byte granule, stores the P = 16 / act_bytes activations of
  // piece c of granule q = g * 64 + j at ((g * (EPG / P) + c) * 64 + j) * P, so
  // that lane j of a wave reads its granules' activations with coalesced
  // loads.  in_sliced: this launch's input rows (x / x_s, or h / h_s) are
  // sliced for the matrix that consumes them; out_sliced: gate/up writes h and
  // h_s sliced for the down matrices of the same sets.
  int32_t in_sliced, out_sliced;
  float* y;                // routed down output rows [slot f][H]
  float* y_s;              // shared down output rows [token][H]
  // optional copies of h (gate/up) in fp32 before any rounding, rows as h and
  // h_s, columns in natural order (a test hook; null: none)
  float* hp;
  float* hp_s;
  // filled in by the launcher
  MatGeo geo, geo_s;
  int32_t rb, nb, rb_s, nb_s;
  // Token mode, for buckets with more rows than one pass of the kernel takes:
  // routed slots are bucket positions (one token of one expert per block) and
  // the shared expert's row blocks are repeated for ntg_s groups of tok_s
  // tokens, so that no block makes a second pass over its weight rows.
  // Otherwise routed slots are active experts and ntg_s = 1, tok_s = n_tok.
  int32_t per_token, tok_s, ntg_s;
};

// One grouped-GEMM launch (prefill-sized buckets, bf16 activations): the
// routed tiles of the buckets and, optionally, the shared expert's token rows.
struct GgArgs {
  ExpertSetDev w, ws;
  int32_t has_shared, H, I, Is, T, top_k;
  const int32_t* entries;    // bucket entries (flat slot f = t * top_k + j)
  const int32_t* tile_e;     // routed m-tiles: expert, first bucket position, rows
  const int32_t* tile_p0;
  const int32_t* tile_n;
  const int32_t* tile_first; // first m-tile of the tile's expert, and its count
  const int32_t* tile_cnt;
  const int32_t* n_tiles;    // routed m-tiles in use (device)
  int32_t max_tiles;         // routed m-tiles in the grid
  const uint16_t* x;         // [T][H] bf16
  const uint16_t* x_p;       // x with each group of 8 in the order 0,4,1,5,2,6,3,7
                             // (read by int4 experts; h of int4 experts is
                             // written in that order too)
  uint16_t* h;               // [bucket position][I] bf16
  uint16_t* h_s;             // [T][Is] bf16
  float* y;                  // [slot f][H]
  float* y_s;                // [T][H]
  // optional fp32 copies of h and h_s before rounding, natural column order
  // (a test hook; null: none)
  float* hp;
  float* hp_s;
  // fp32 row sums of the bf16 activation rows of int4 experts (the int4
  // operand carries an offset that the epilogue removes with them)
  const float* rs_x;         // [T]       rows of x
  const float* rs_h;         // [T * k]   rows of h
  const float* rs_hs;        // [T]       rows of the shared expert's h
  // filled in by the launcher
  int32_t s_tiles, nt_r, nt_s;
};

// ------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  Shapes are validated by the
// caller (moe_capi.cpp).

hipError_t launch_rmsnorm(const float* x, float* out, int32_t T, int32_t H, float eps,
                          hipStream_t s);
// Router logits; for T <= kDecodeTokens the same launch also writes the
// sliced copies that sr asks for (larger T: launch_slice_rows).
hipError_t launch_router_logits(const float* w_router, const void* x, int act_bf16, int32_t T,
                                int32_t H, int32_t E, double* z, const SliceReq& sr,
                                hipStream_t s, double* zpart = nullptr, int64_t zpart_elems = 0);
// Copies of the T activation rows in the sliced layouts of up to two weight
// formats (epg 0 or dst null: skipped).
hipError_t launch_slice_rows(const void* x, int act_bf16, int32_t T, int32_t K, int32_t epg_a,
                             void* dst_a, int32_t epg_b, void* dst_b, hipStream_t s);
SelectParams select_params(const moe_layer_desc& d);
hipError_t launch_router_select(const moe_layer_desc& d, const double* z, const float* bias,
                                int32_t T, int32_t* topk_idx, float* topk_w, hipStream_t s);
hipError_t launch_bucket(int32_t T, int32_t K, int32_t E, const int32_t* topk_idx,
                         int32_t* counts, int32_t* offsets, int32_t* entries, int32_t* inverse,
                         int32_t* active, int32_t* n_active, hipStream_t s);
// Gate/up + SwiGLU (down = false) or the down projection (down = true) of
// the routed slots and, when a.has_shared, the shared expert, in one launch.
// max_rows_per_slot bounds the rows of any slot (1 selects the one-row path).
hipError_t launch_gemv(GemvArgs a, bool down, int dtype, int shared_dtype, int act_bf16,
                       int max_rows_per_slot, hipStream_t s);
bool make_geo(int dtype, int32_t K, MatGeo& g);
// A shared-expert-only GEMV launch (a.has_shared, no routed slots) whose
// leading p.blocks blocks run the routing work p (decode).
hipError_t launch_gemv_pre(GemvArgs a, const PreArgs& p, bool down, int shared_dtype,
                           int act_bf16, hipStream_t s);
// Whether launch_gemv_pre covers the layer: sigmoid router with at most 256
// experts, and a shared set in a format with LDS-ring kernels for its gate/up
// (input H) and down (input Is) rows.
bool gemv_pre_supported(const moe_layer_desc& d, int32_t Is);
// Decode-sized routing: selection for T <= kDecodeTokens tokens and the
// bucketing, in one single-block launch.
hipError_t launch_select_bucket(const moe_layer_desc& d, const double* z, const float* bias,
                                int32_t T, int32_t* topk_idx, float* topk_w, int32_t* counts,
                                int32_t* offsets, int32_t* entries, int32_t* inverse,
                                int32_t* active, int32_t* n_active, hipStream_t s,
                                const SlotTables& tb = SlotTables{});
// out[t] = sum_j w[t][j] * Y[t*k + j] + (S ? S[t] : 0) (+ residual[t] when given;
// then y_copy[t] receives the MoE output without the residual).
hipError_t launch_combine(const float* Y, const int32_t* topk_idx, const float* topk_w,
                          const float* S, int32_t T, int32_t K, int32_t H, const float* residual,
                          float* out, float* y_copy, hipStream_t s);
hipError_t launch_requant_fp8_int4(const uint8_t* fp8, const float* block_scales, int32_t rows,
                                   int32_t cols, int32_t block, uint8_t* codes, float* scales,
                                   hipStream_t s);
bool requant_supported(int32_t cols, int32_t block);
// Device address of the library's own workspace on the device that `stream`
// runs on (kNoAllocScratchBytes bytes; looked up once per device).
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);
hipError_t launch_dequant(int dtype, const void* codes, const float* scales, int32_t cols,
                          int32_t row0, int32_t n_rows, float* out, uint16_t* out_bf16,
                          hipStream_t s);

// One-token decode: the routed gate/up launch whose blocks each run the
// selection and grouping themselves (k_gemv_sel.hip), block 0 writing them
// out (p: the selection parameters, logits and outputs, as for the selection
// launch); whether the layer's shapes are compiled.
bool gemv_sel_supported(const moe_layer_desc& d, int32_t T);
hipError_t launch_gemv_sel(GemvArgs a, const PreArgs& p, int dtype, int act_bf16, hipStream_t s);

// One-token decode: the routed and shared down projections and the combine
// in one launch (k_down_fused.hip); whether the layer's shapes are covered.
struct DownFusedArgs;
bool down_fused_supported(const moe_layer_desc& d, int32_t T);
hipError_t launch_down_fused(const moe_layer_desc& d, DownFusedArgs a, int act_bf16,
                             hipStream_t s);

// Grouped GEMM: whether a layer qualifies, the routed m-tile bound for T
// tokens, the tile list from the buckets, and the launch.
bool ggemm_supported(const moe_layer_desc& d);
int32_t ggemm_max_tiles(int32_t T, int32_t K, int32_t E);
hipError_t launch_make_tiles(const int32_t* offsets, const int32_t* active, const int32_t* n_active,
                             int32_t* tile_e, int32_t* tile_p0, int32_t* tile_n,
                             int32_t* tile_first, int32_t* tile_cnt, int32_t* n_tiles,
                             hipStream_t s);
hipError_t launch_ggemm(GgArgs a, bool down, int dtype, int shared_dtype, hipStream_t s);
// The shared expert's dense GEMMs for prefill batches (shared_blaslt.cpp):
// D[M][N] (fp32, row-major) = B[M][K] (bf16 rows) x A[N][K]^T (bf16 rows).
// shared_gemm_ready tells whether both of a layer's shapes (gate/up N1 x K1,
// down N2 x K2) have a handle and an algorithm on the stream's device
// (prepared on first use outside graph capture).
constexpr int kSharedDenseMinTokens = 256;
bool shared_gemm_ready(hipStream_t s, int M, int N1, int K1, int N2, int K2);
hipError_t shared_gemm(int M, int N, int K, const void* A, const void* B, float* D, hipStream_t s);
// h = bf16(silu(GU[:, :Is]) * GU[:, Is:]) over T fp32 rows of 2 Is (k_misc.hip)
hipError_t launch_swiglu_rows(const float* gu, int32_t T, int32_t Is, uint16_t* h, float* hp,
                              hipStream_t s);
hipError_t launch_rowsum_bf16(const uint16_t* rows, int32_t n, int32_t K, float* out,
                              uint16_t* perm, hipStream_t s);

// Whether the GEMV kernels cover an input length K of this dtype: K must be
// a whole number of 64-granule chunks, or a power-of-two number of granules
// below 64 (granule: 32 int4/int2 codes or 8 bf16 values).
bool gemv_supported(int dtype, int32_t K);
// Whether a routed set (dtype, input K) and the shared set (sdtype, input Ks)
// can share one launch: both covered, with the same per-lane slice geometry.
bool gemv_pair_supported(int dtype, int32_t K, int sdtype, int32_t Ks);
// Whether the expert GEMV of this format streams rows of length K through the
// LDS ring (rows of >= 64 granules of 16 bytes), the path that reads sliced
// activation rows.
bool gemv_ring(int dtype, int32_t K);

// Moves 16-byte piece p of the sliced copy (epg) of a row of K activations of
// ab bytes from the row-major row.
__device__ __forceinline__ void slice_piece(const uint8_t* row, uint8_t* dst_row, int64_t p,
                                            int epg, int ab) {
  const int P = 16 / ab, ppc = epg / P;
  const int64_t j = p & 63, gc = p >> 6;
  const int64_t g = gc / ppc, c = gc - g * ppc;
  const int64_t e0 = (g * 64 + j) * epg + c * P;
  *reinterpret_cast<uint4*>(dst_row + p * 16) = *reinterpret_cast<const uint4*>(row + e0 * ab);
}

// Element index of activation e of a row in the sliced layout (see GemvArgs).
__host__ __device__ __forceinline__ int64_t sliced_index(int64_t e, int epg, int act_bytes) {
  const int P = 16 / act_bytes;
  const int64_t q = e / epg;
  const int64_t g = q >> 6, j = q & 63;
  const int64_t c = (e % epg) / P, u = e % P;
  return ((g * (epg / P) + c) * 64 + j) * P + u;
}

}  // namespace moe
