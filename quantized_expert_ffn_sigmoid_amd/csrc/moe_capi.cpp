// moe_capi.cpp -- the C ABI of include/moe.h: host-side validation, workspace
// carving and the launch sequence of the routed MoE layer on gfx950.
//
// No call allocates, frees or synchronises; every launch goes on the caller's
// stream, so a decode step can be captured into a HIP graph by the caller.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "down_fused.h"
#include "moe.h"
#include "moe_internal.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_is_weight(int32_t t) {
  return t == MOE_I4 || t == MOE_I2 || t == MOE_I8 || t == MOE_BF16;
}

// Descriptor consistency (MOE_EINVAL) and kernel coverage (MOE_EUNSUPPORTED).
// The decode-sized expert path (GEMV kernels) covers the layer's shapes.
bool gemv_layer_ok(const moe_layer_desc& d) {
  if (!gemv_supported(d.expert_dtype, d.hidden) || !gemv_supported(d.expert_dtype, d.inter))
    return false;
  if (d.n_shared > 0 &&
      (!gemv_pair_supported(d.expert_dtype, d.hidden, d.shared_dtype, d.hidden) ||
       !gemv_pair_supported(d.expert_dtype, d.inter, d.shared_dtype, d.inter * d.n_shared)))
    return false;
  return true;
}

// layer: also require that one expert path covers the whole layer (routed
// and shared sets together); single-expert calls check their own set only.
moe_status check_desc(const moe_layer_desc* d, bool layer = true) {
  if (!d) return MOE_EINVAL;
  if (d->hidden <= 0 || d->inter <= 0 || d->n_experts <= 0 || d->top_k <= 0) return MOE_EINVAL;
  if (d->top_k > d->n_experts) return MOE_EINVAL;
  if (d->router != MOE_ROUTER_SIGMOID_NOAUX_TC && d->router != MOE_ROUTER_SOFTMAX_TOPK)
    return MOE_EINVAL;
  if (d->router == MOE_ROUTER_SIGMOID_NOAUX_TC) {
    if (d->n_group <= 0 || d->n_experts % d->n_group != 0) return MOE_EINVAL;
    if (d->topk_group <= 0 || d->topk_group > d->n_group) return MOE_EINVAL;
    if ((int64_t)d->topk_group * (d->n_experts / d->n_group) < d->top_k) return MOE_EINVAL;
  }
  if (!dtype_is_weight(d->expert_dtype)) return MOE_EINVAL;
  if (d->act_dtype != MOE_F32 && d->act_dtype != MOE_BF16) return MOE_EINVAL;
  if (d->n_shared < 0 || d->n_shared > 1) return MOE_EINVAL;
  if (d->n_shared > 0 && !dtype_is_weight(d->shared_dtype)) return MOE_EINVAL;
  if (!(d->top_p >= 0.0f)) return MOE_EINVAL;   // also rejects NaN
  // kernel coverage
  if (d->n_experts > kMaxExperts || d->top_k > kMaxTopK) return MOE_EUNSUPPORTED;
  if (d->router == MOE_ROUTER_SIGMOID_NOAUX_TC && d->n_group > 64) return MOE_EUNSUPPORTED;
  if (d->hidden % 32 != 0) return MOE_EUNSUPPORTED;
  // a layer is accepted when either expert path covers it; calls whose batch
  // size selects an uncovered path fail with MOE_EUNSUPPORTED
  if (layer && !gemv_layer_ok(*d) && !ggemm_supported(*d)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

moe_status check_set(const moe_expert_set* s, int32_t dtype) {
  if (!s) return MOE_EINVAL;
  if (!s->gate_up || !s->down || !aligned16(s->gate_up) || !aligned16(s->down)) return MOE_EINVAL;
  if ((s->gate_up_stride & 15) || (s->down_stride & 15)) return MOE_EINVAL;
  if (s->gate_up_stride < 0 || s->down_stride < 0) return MOE_EINVAL;
  if (dtype != MOE_BF16) {
    if (!s->gate_up_scale || !s->down_scale) return MOE_EINVAL;
    if (!aligned16(s->gate_up_scale) || !aligned16(s->down_scale)) return MOE_EINVAL;
    if ((s->gate_up_scale_stride & 15) || (s->down_scale_stride & 15)) return MOE_EINVAL;
  }
  return MOE_OK;
}

ExpertSetDev dev_set(const moe_expert_set& s) {
  ExpertSetDev v;
  v.gu = static_cast<const uint8_t*>(s.gate_up);
  v.gu_stride = s.gate_up_stride;
  v.gus = reinterpret_cast<const uint8_t*>(s.gate_up_scale);
  v.gus_stride = s.gate_up_scale_stride;
  v.dn = static_cast<const uint8_t*>(s.down);
  v.dn_stride = s.down_stride;
  v.dns = reinterpret_cast<const uint8_t*>(s.down_scale);
  v.dns_stride = s.down_scale_stride;
  return v;
}

// Elements per 16-byte granule of a weight format (the unit of the sliced
// activation layout).
int32_t epg_of(int32_t dtype) { return dtype == MOE_BF16 ? 8 : 32; }

// Workspace carve for n tokens.  Every region is 256-byte aligned.
struct Carve {
  size_t z, idx, w, counts, offsets, entries, inverse, active, n_active, h, h_sh, Y, S, xn, yl,
      xs, xs_sh, tiles, rs, xp, slot_tab, pos_e, zsc, total;
};

Carve carve(const moe_layer_desc& d, int64_t T) {
  Carve c{};
  const int64_t E = d.n_experts, K = d.top_k, H = d.hidden, I = d.inter;
  const int64_t Ish = (int64_t)d.inter * d.n_shared;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  c.z = take(sizeof(double) * T * E);
  c.idx = take(sizeof(int32_t) * T * K);
  c.w = take(sizeof(float) * T * K);
  c.counts = take(sizeof(int32_t) * E);
  c.offsets = take(sizeof(int32_t) * (E + 1));
  c.entries = take(sizeof(int32_t) * T * K);
  c.inverse = take(sizeof(int32_t) * T * K);
  c.active = take(sizeof(int32_t) * E);
  c.n_active = take(sizeof(int32_t));
  c.h = take(sizeof(float) * T * K * I);
  c.h_sh = take(sizeof(float) * T * (Ish > I ? Ish : I));
  c.Y = take(sizeof(float) * T * K * H);
  c.S = take(sizeof(float) * T * H);
  c.xn = take(sizeof(float) * T * H);
  c.yl = take(sizeof(float) * T * H);
  c.xs = take(sizeof(float) * T * H);
  c.xs_sh = take(sizeof(float) * T * H);
  c.tiles = take(sizeof(int32_t) * (5 * (size_t)ggemm_max_tiles((int32_t)T, (int32_t)K, (int32_t)E) + 1));
  c.rs = take(sizeof(float) * (size_t)T * (K + 2));
  c.xp = take(sizeof(uint16_t) * (size_t)T * H);
  c.slot_tab = take(sizeof(int32_t) * kSlotRec * (size_t)(T * K < E ? T * K : E));
  c.pos_e = take(sizeof(int32_t) * (size_t)T * K);
  c.zsc = take(sizeof(double) * 2 * (size_t)(T <= kDecodeTokens ? T : 0) * E);
  c.total = o;
  return c;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

void record(const moe_launch_opts* opts, int stage, int end, hipStream_t s) {
  if (opts && opts->events) {
    hipEvent_t ev = static_cast<hipEvent_t>(opts->events[2 * stage + end]);
    if (!ev) return;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs == hipStreamCaptureStatusActive)
      (void)hipEventRecordWithFlags(ev, s, hipEventRecordExternal);
    else
      (void)hipEventRecord(ev, s);
  }
}

#define MOE_TRY(expr)                       \
  do {                                      \
    if ((expr) != hipSuccess) return MOE_EHIP; \
  } while (0)

// The layer: out = combine(...) (+ residual when given; y_copy then receives
// the layer output).  Arguments already validated.
moe_status layer_impl(const moe_layer_desc& d, const moe_layer_weights& w, const void* x,
                      int32_t T, float* out, int32_t* idx_out, float* w_out, void* ws,
                      const float* residual, float* y_copy, hipStream_t s,
                      const moe_launch_opts* opts) {
  const Carve c = carve(d, T);
  const int32_t E = d.n_experts, K = d.top_k, H = d.hidden, I = d.inter;
  const int act_bf16 = d.act_dtype == MOE_BF16;
  int32_t* idx = idx_out ? idx_out : at<int32_t>(ws, c.idx);
  float* tw = w_out ? w_out : at<float>(ws, c.w);
  double* z = at<double>(ws, c.z);
  int32_t* counts = at<int32_t>(ws, c.counts);
  int32_t* offsets = at<int32_t>(ws, c.offsets);
  int32_t* entries = at<int32_t>(ws, c.entries);
  int32_t* inverse = at<int32_t>(ws, c.inverse);
  int32_t* active = at<int32_t>(ws, c.active);
  int32_t* n_active = at<int32_t>(ws, c.n_active);
  // decode grouping also writes per-slot records for the expert kernels
  SlotTables tb;
  if (T <= kDecodeTokens) {
    tb.slot_tab = at<int32_t>(ws, c.slot_tab);
    tb.n_tab = T * K < E ? T * K : E;
    tb.pos_e = at<int32_t>(ws, c.pos_e);
  }
  void* h = at<void>(ws, c.h);
  void* h_sh = at<void>(ws, c.h_sh);
  float* Y = at<float>(ws, c.Y);
  float* S = at<float>(ws, c.S);

  // Sliced activation rows (a coalesced per-lane layout) for the expert
  // kernels that stream their weights through the LDS ring.
  const bool has_sh = d.n_shared > 0;
  const int32_t Ish = I * (has_sh ? d.n_shared : 1);
  const bool gu_ring = gemv_ring(d.expert_dtype, H) && (!has_sh || gemv_ring(d.shared_dtype, H));
  const bool dn_ring = gemv_ring(d.expert_dtype, I) && (!has_sh || gemv_ring(d.shared_dtype, Ish));
  const int epg_r = epg_of(d.expert_dtype), epg_s = has_sh ? epg_of(d.shared_dtype) : 0;
  void* xs = at<void>(ws, c.xs);
  void* xs_sh = epg_s && epg_s != epg_r ? at<void>(ws, c.xs_sh) : xs;

  const bool use_gg = T > kDecodeTokens && ggemm_supported(d);
  if (!use_gg && !gemv_layer_ok(d)) return MOE_EUNSUPPORTED;
  const bool fused_route = T <= kDecodeTokens;
  // Decode with a shared expert: its launches carry the routing work in their
  // leading blocks (the shared expert does not depend on the routing), and
  // the routed launches follow.  The shared gate/up then reads x as it is.
  const bool pre = !use_gg && fused_route && gu_ring && dn_ring && gemv_pre_supported(d, Ish);
  // one token on the ring kernels: the down projections (routed and shared)
  // and the combine run as one launch that writes out directly
  const bool fused_dn = !use_gg && T == 1 && gu_ring && dn_ring && down_fused_supported(d, T);
  DownFusedArgs fa{};
  if (fused_dn) {
    fa.w = dev_set(w.routed);
    if (has_sh) fa.ws = dev_set(w.shared);
    fa.has_shared = has_sh;
    fa.H = H;
    fa.I = I;
    fa.Is = Ish;
    fa.slot_tab = tb.slot_tab;
    fa.n_slots = tb.n_tab;
    fa.topk_w = tw;
    fa.h = h;
    fa.h_s = h_sh;
    fa.residual = residual;
    fa.out = out;
    fa.y_copy = y_copy;
  }
  SliceReq sr{};
  if (gu_ring && !use_gg) {
    sr.epg_a = epg_r;
    sr.dst_a = xs;
    if (xs_sh != xs && !pre) {
      sr.epg_b = epg_s;
      sr.dst_b = xs_sh;
    }
  }

  GemvArgs g{};
  g.w = dev_set(w.routed);
  if (has_sh) g.ws = dev_set(w.shared);
  g.src.routed = 1;
  g.src.active = active;
  g.src.n_active = n_active;
  g.src.offsets = offsets;
  g.src.entries = entries;
  g.src.slot_tab = tb.slot_tab;
  g.src.pos_e = tb.pos_e;
  g.src.top_k = K;
  g.has_shared = has_sh;
  g.n_tok = T;
  g.H = H;
  g.I = I;
  g.Is = Ish;
  g.n_slots = (int64_t)T * K < E ? T * K : E;
  g.x = gu_ring ? xs : x;
  g.x_s = gu_ring ? xs_sh : nullptr;
  g.h = h;
  g.h_s = h_sh;
  g.y = Y;
  g.y_s = S;
  g.in_sliced = gu_ring;
  g.out_sliced = gu_ring && dn_ring;
  float* hp = opts ? opts->h_f32 : nullptr;
  g.hp = hp;
  g.hp_s = hp ? hp + (int64_t)T * K * I : nullptr;

  // One token with the fused down launch: the routed gate/up blocks run the
  // selection and grouping themselves (no launch of its own).
  // (outside the decode launches that carry the router, a shared expert's
  // gate/up shares the routed launch, which this variant does not hold)
  const bool sel_inline = fused_dn && (pre || !has_sh) && gemv_sel_supported(d, T);
  PreArgs sel{};
  // the selection reads the scores the logits launch formed (sigmoid router
  // with the logits in the shared expert's launch)
  double* zsc = (sel_inline && pre && d.router == MOE_ROUTER_SIGMOID_NOAUX_TC)
                    ? at<double>(ws, c.zsc) : nullptr;
  if (sel_inline) {
    sel.sp = select_params(d);
    sel.sp.zsc = zsc;
    sel.T = T;
    sel.zin = z;
    sel.bias = w.bias;
    sel.idx = idx;
    sel.w = tw;
    sel.counts = counts;
    sel.offsets = offsets;
    sel.entries = entries;
    sel.inverse = inverse;
    sel.active = active;
    sel.n_active = n_active;
    sel.tb = tb;
    // a bf16 shared expert of intermediate size kSdnIs: its down projection
    // runs in the gate/up launch, beside the selection, and the down launch
    // adds its output
    if (pre && has_sh && d.shared_dtype == MOE_BF16 && Ish == kSdnIs) {
      sel.H = H;
      sel.sdn = fa.ws.dn;
      sel.sdn_h = h_sh;
      sel.sdn_out = S;
      fa.s_pre = S;
    }
  }

  if (pre) {
    record(opts, MOE_STAGE_ROUTE, 0, s);
    GemvArgs gs = g;
    gs.x = x;
    gs.x_s = nullptr;
    gs.in_sliced = 0;
    PreArgs p{};
    p.kind = kPreLogits;
    p.blocks = E;
    p.w_router = w.w_router;
    p.x = x;
    p.act_bf16 = act_bf16;
    p.T = T;
    p.H = H;
    p.E = E;
    p.z = z;
    p.sr = sr;
    p.zsc = zsc;
    p.zbias = w.bias;
    MOE_TRY(launch_gemv_pre(gs, p, false, d.shared_dtype, act_bf16, s));
    if (fused_dn) {
      // the shared down projection joins the routed ones in the fused launch;
      // the selection and grouping run in the routed gate/up blocks (or, for
      // shapes that launch does not compile, in one block of their own)
      if (!sel_inline)
        MOE_TRY(launch_select_bucket(d, z, w.bias, T, idx, tw, counts, offsets, entries, inverse,
                                     active, n_active, s, tb));
      record(opts, MOE_STAGE_ROUTE, 1, s);
      record(opts, MOE_STAGE_BUCKET, 0, s);
      record(opts, MOE_STAGE_BUCKET, 1, s);
      g.has_shared = 0;
      record(opts, MOE_STAGE_GATE_UP, 0, s);
      if (sel_inline)
        MOE_TRY(launch_gemv_sel(g, sel, d.expert_dtype, act_bf16, s));
      else
        MOE_TRY(launch_gemv(g, false, d.expert_dtype, d.shared_dtype, act_bf16, T, s));
      record(opts, MOE_STAGE_GATE_UP, 1, s);
      record(opts, MOE_STAGE_DOWN, 0, s);
      MOE_TRY(launch_down_fused(d, fa, act_bf16, s));
      record(opts, MOE_STAGE_DOWN, 1, s);
      record(opts, MOE_STAGE_COMBINE, 0, s);
      record(opts, MOE_STAGE_COMBINE, 1, s);
      return MOE_OK;
    }
    gs.in_sliced = g.out_sliced;
    p = PreArgs{};
    p.kind = kPreSelect;
    p.blocks = 1;
    p.sp = select_params(d);
    p.T = T;
    p.zin = z;
    p.bias = w.bias;
    p.idx = idx;
    p.w = tw;
    p.counts = counts;
    p.offsets = offsets;
    p.entries = entries;
    p.inverse = inverse;
    p.active = active;
    p.n_active = n_active;
    p.tb = tb;
    MOE_TRY(launch_gemv_pre(gs, p, true, d.shared_dtype, act_bf16, s));
    record(opts, MOE_STAGE_ROUTE, 1, s);
    record(opts, MOE_STAGE_BUCKET, 0, s);
    record(opts, MOE_STAGE_BUCKET, 1, s);
    g.has_shared = 0;
    record(opts, MOE_STAGE_GATE_UP, 0, s);
    MOE_TRY(launch_gemv(g, false, d.expert_dtype, d.shared_dtype, act_bf16, T, s));
    record(opts, MOE_STAGE_GATE_UP, 1, s);
    record(opts, MOE_STAGE_DOWN, 0, s);
    g.in_sliced = g.out_sliced;
    MOE_TRY(launch_gemv(g, true, d.expert_dtype, d.shared_dtype, act_bf16, T, s));
    record(opts, MOE_STAGE_DOWN, 1, s);
    record(opts, MOE_STAGE_COMBINE, 0, s);
    MOE_TRY(launch_combine(Y, idx, tw, S, T, K, H, residual, out, y_copy, s));
    record(opts, MOE_STAGE_COMBINE, 1, s);
    return MOE_OK;
  }

  record(opts, MOE_STAGE_ROUTE, 0, s);
  // the partial sums of a split-K router GEMM use the Y area, unused until
  // the down projections
  MOE_TRY(launch_router_logits(w.w_router, x, act_bf16, T, H, E, z, sr, s,
                               reinterpret_cast<double*>(Y), (int64_t)T * K * H / 2));
  if (fused_route && !sel_inline)
    MOE_TRY(launch_select_bucket(d, z, w.bias, T, idx, tw, counts, offsets, entries, inverse,
                                 active, n_active, s, tb));
  else if (!fused_route)
    MOE_TRY(launch_router_select(d, z, w.bias, T, idx, tw, s));
  record(opts, MOE_STAGE_ROUTE, 1, s);

  record(opts, MOE_STAGE_BUCKET, 0, s);
  if (!fused_route)
    MOE_TRY(launch_bucket(T, K, E, idx, counts, offsets, entries, inverse, active, n_active, s));
  record(opts, MOE_STAGE_BUCKET, 1, s);

  if (use_gg) {
    // prefill-sized buckets: grouped GEMM on the matrix cores
    const int32_t mt = ggemm_max_tiles(T, K, E);
    int32_t* tiles = at<int32_t>(ws, c.tiles);
    GgArgs q{};
    q.w = dev_set(w.routed);
    if (has_sh) q.ws = dev_set(w.shared);
    q.has_shared = has_sh;
    q.H = H;
    q.I = I;
    q.Is = Ish;
    q.T = T;
    q.top_k = K;
    q.entries = entries;
    q.tile_e = tiles;
    q.tile_p0 = tiles + mt;
    q.tile_n = tiles + 2 * mt;
    q.tile_first = tiles + 3 * mt;
    q.tile_cnt = tiles + 4 * mt;
    q.n_tiles = tiles + 5 * mt;
    q.max_tiles = mt;
    q.x = static_cast<const uint16_t*>(x);
    q.h = static_cast<uint16_t*>(h);
    q.h_s = static_cast<uint16_t*>(h_sh);
    q.y = Y;
    q.y_s = S;
    q.hp = g.hp;
    q.hp_s = g.hp_s;
    float* rs = at<float>(ws, c.rs);
    q.rs_x = rs;
    q.rs_h = rs + T;
    q.rs_hs = rs + (int64_t)T * (K + 1);
    const bool any_i4 = d.expert_dtype == MOE_I4 || (has_sh && d.shared_dtype == MOE_I4);
    // A bf16 shared expert over a large batch is two plain dense GEMMs: they
    // go to the platform's GEMM library (its gate/up output, fp32 [T][2 Is],
    // in the Y area, which the routed down projection fills only later).
    const bool sh_dense = has_sh && d.shared_dtype == MOE_BF16 && T >= kSharedDenseMinTokens &&
                          (int64_t)K * H >= 2 * (int64_t)Ish &&
                          shared_gemm_ready(s, T, 2 * Ish, H, H, Ish);
    GgArgs qr = q;
    if (sh_dense) qr.has_shared = 0;
    MOE_TRY(launch_make_tiles(offsets, active, n_active, tiles, tiles + mt, tiles + 2 * mt,
                              tiles + 3 * mt, tiles + 4 * mt, tiles + 5 * mt, s));
    record(opts, MOE_STAGE_GATE_UP, 0, s);
    q.x_p = qr.x_p = at<uint16_t>(ws, c.xp);
    if (any_i4) MOE_TRY(launch_rowsum_bf16(q.x, T, H, rs, at<uint16_t>(ws, c.xp), s));
    MOE_TRY(launch_ggemm(qr, false, d.expert_dtype, d.shared_dtype, s));
    if (sh_dense) {
      MOE_TRY(shared_gemm(T, 2 * Ish, H, w.shared.gate_up, x, Y, s));
      MOE_TRY(launch_swiglu_rows(Y, T, Ish, q.h_s, q.hp_s, s));
    }
    record(opts, MOE_STAGE_GATE_UP, 1, s);
    record(opts, MOE_STAGE_DOWN, 0, s);
    if (d.expert_dtype == MOE_I4) MOE_TRY(launch_rowsum_bf16(q.h, T * K, I, rs + T, nullptr, s));
    if (has_sh && d.shared_dtype == MOE_I4)
      MOE_TRY(launch_rowsum_bf16(q.h_s, T, Ish, rs + (int64_t)T * (K + 1), nullptr, s));
    MOE_TRY(launch_ggemm(qr, true, d.expert_dtype, d.shared_dtype, s));
    if (sh_dense) MOE_TRY(shared_gemm(T, H, Ish, w.shared.down, q.h_s, S, s));
    record(opts, MOE_STAGE_DOWN, 1, s);
    record(opts, MOE_STAGE_COMBINE, 0, s);
    MOE_TRY(launch_combine(Y, idx, tw, has_sh ? S : nullptr, T, K, H, residual, out, y_copy, s));
    record(opts, MOE_STAGE_COMBINE, 1, s);
    return MOE_OK;
  }

  record(opts, MOE_STAGE_GATE_UP, 0, s);
  if (sel_inline)
    MOE_TRY(launch_gemv_sel(g, sel, d.expert_dtype, act_bf16, s));
  else
    MOE_TRY(launch_gemv(g, false, d.expert_dtype, d.shared_dtype, act_bf16, T, s));
  record(opts, MOE_STAGE_GATE_UP, 1, s);

  if (fused_dn) {
    record(opts, MOE_STAGE_DOWN, 0, s);
    MOE_TRY(launch_down_fused(d, fa, act_bf16, s));
    record(opts, MOE_STAGE_DOWN, 1, s);
    record(opts, MOE_STAGE_COMBINE, 0, s);
    record(opts, MOE_STAGE_COMBINE, 1, s);
    return MOE_OK;
  }
  record(opts, MOE_STAGE_DOWN, 0, s);
  g.in_sliced = g.out_sliced;
  MOE_TRY(launch_gemv(g, true, d.expert_dtype, d.shared_dtype, act_bf16, T, s));
  record(opts, MOE_STAGE_DOWN, 1, s);

  record(opts, MOE_STAGE_COMBINE, 0, s);
  MOE_TRY(launch_combine(Y, idx, tw, d.n_shared > 0 ? S : nullptr, T, K, H, residual, out, y_copy,
                         s));
  record(opts, MOE_STAGE_COMBINE, 1, s);
  return MOE_OK;
}

moe_status check_layer_args(const moe_layer_desc* d, const moe_layer_weights* w) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (!w || !w->w_router || !aligned16(w->w_router)) return MOE_EINVAL;
  if (w->bias && !aligned16(w->bias)) return MOE_EINVAL;
  st = check_set(&w->routed, d->expert_dtype);
  if (st != MOE_OK) return st;
  if (d->n_shared > 0) {
    st = check_set(&w->shared, d->shared_dtype);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_layer_desc* d, int32_t n_tokens) {
  if (check_desc(d, false) != MOE_OK || n_tokens < 0) return 0;
  return carve(*d, n_tokens > 0 ? n_tokens : 1).total;
}

moe_status moe_route(const moe_layer_desc* d, const float* w_router, const float* bias,
                     const void* x, int32_t n_tokens, int32_t* topk_idx, float* topk_w, void* ws,
                     size_t ws_bytes, void* stream) {
  moe_status st = check_desc(d, false);   // routing only: no expert kernels involved
  if (st != MOE_OK) return st;
  if (n_tokens < 0) return MOE_EINVAL;
  if (n_tokens == 0) return MOE_OK;
  if (!w_router || !x || !topk_idx || !topk_w || !ws) return MOE_EINVAL;
  if (!aligned16(w_router) || !aligned16(x) || (bias && !aligned16(bias)) || !aligned16(ws))
    return MOE_EINVAL;
  if (ws_bytes < moe_workspace_bytes(d, n_tokens)) return MOE_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Carve c = carve(*d, n_tokens);
  double* z = at<double>(ws, c.z);
  if (launch_router_logits(w_router, x, d->act_dtype == MOE_BF16, n_tokens, d->hidden,
                           d->n_experts, z, SliceReq{}, s, at<double>(ws, c.Y),
                           (int64_t)n_tokens * d->top_k * d->hidden / 2) != hipSuccess)
    return MOE_EHIP;
  if (launch_router_select(*d, z, bias, n_tokens, topk_idx, topk_w, s) != hipSuccess)
    return MOE_EHIP;
  return MOE_OK;
}

moe_status moe_bucket(int32_t n_tokens, int32_t top_k, int32_t n_experts, const int32_t* topk_idx,
                      int32_t* counts, int32_t* offsets, int32_t* entries, int32_t* inverse,
                      int32_t* active, int32_t* n_active, void* ws, size_t ws_bytes,
                      void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (n_tokens < 0 || top_k <= 0 || n_experts <= 0) return MOE_EINVAL;
  if (n_experts > kMaxExperts) return MOE_EUNSUPPORTED;
  if (!counts || !offsets || !active || !n_active) return MOE_EINVAL;
  if (n_tokens > 0 && (!topk_idx || !entries || !inverse)) return MOE_EINVAL;
  if ((int64_t)n_tokens * top_k > INT32_MAX) return MOE_EUNSUPPORTED;
  if (launch_bucket(n_tokens, top_k, n_experts, topk_idx, counts, offsets, entries, inverse,
                    active, n_active, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_EHIP;
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_layer_desc* d, const moe_expert_set* set, int32_t shared,
                          int32_t expert, const void* x, const int32_t* rows, int32_t n_rows,
                          int32_t row_div, float* y, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_desc(d, false);
  if (st != MOE_OK) return st;
  if (n_rows < 0 || row_div <= 0) return MOE_EINVAL;
  if (shared && (d->n_shared <= 0 || expert != 0)) return MOE_EINVAL;
  if (!shared && (expert < 0 || expert >= d->n_experts)) return MOE_EINVAL;
  if (n_rows == 0) return MOE_OK;
  const int32_t dtype = shared ? d->shared_dtype : d->expert_dtype;
  st = check_set(set, dtype);
  if (st != MOE_OK) return st;
  if (!x || !y || !ws || !aligned16(x) || !aligned16(y) || !aligned16(ws)) return MOE_EINVAL;
  if (ws_bytes < moe_workspace_bytes(d, n_rows)) return MOE_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t I = shared ? d->inter * d->n_shared : d->inter;
  const int act_bf16 = d->act_dtype == MOE_BF16;
  if (!gemv_supported(dtype, d->hidden) || !gemv_supported(dtype, I)) return MOE_EUNSUPPORTED;
  GemvArgs g{};
  g.w = dev_set(*set);
  g.src.routed = 0;
  g.src.fixed_expert = expert;
  g.src.rows = rows;
  g.src.n_rows = n_rows;
  g.src.row_div = row_div;
  g.has_shared = 0;
  g.H = d->hidden;
  g.I = I;
  g.Is = I;
  g.n_slots = 1;
  g.x = x;
  g.h = at<void>(ws, carve(*d, n_rows).h);
  g.y = y;
  g.in_sliced = 0;
  g.out_sliced = gemv_ring(dtype, d->hidden) && gemv_ring(dtype, I);
  if (launch_gemv(g, false, dtype, dtype, act_bf16, n_rows, s) != hipSuccess) return MOE_EHIP;
  g.src.rows = nullptr;   // down reads h rows 0..n_rows-1 and writes y rows 0..n_rows-1
  g.src.row_div = 1;
  g.in_sliced = g.out_sliced;
  if (launch_gemv(g, true, dtype, dtype, act_bf16, n_rows, s) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

moe_status moe_layer_forward_ex(const moe_layer_desc* d, const moe_layer_weights* w,
                                const void* x, int32_t n_tokens, float* out,
                                int32_t* topk_idx_out, float* topk_w_out, void* ws,
                                size_t ws_bytes, void* stream, const moe_launch_opts* opts) {
  moe_status st = check_layer_args(d, w);
  if (st != MOE_OK) return st;
  if (n_tokens < 0) return MOE_EINVAL;
  if (n_tokens == 0) return MOE_OK;
  if (!x || !out || !ws || !aligned16(x) || !aligned16(out) || !aligned16(ws)) return MOE_EINVAL;
  if (ws_bytes < moe_workspace_bytes(d, n_tokens)) return MOE_EWORKSPACE;
  return layer_impl(*d, *w, x, n_tokens, out, topk_idx_out, topk_w_out, ws, nullptr, nullptr,
                    static_cast<hipStream_t>(stream), opts);
}

moe_status moe_layer_forward(const moe_layer_desc* d, const moe_layer_weights* w, const void* x,
                             int32_t n_tokens, float* out, int32_t* topk_idx_out,
                             float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  return moe_layer_forward_ex(d, w, x, n_tokens, out, topk_idx_out, topk_w_out, ws, ws_bytes,
                              stream, nullptr);
}

moe_status moe_layer_forward_noalloc(const moe_layer_desc* d, const moe_layer_weights* w,
                                     const void* x, int32_t n_tokens, float* out,
                                     int32_t* topk_idx_out, float* topk_w_out, void* stream) {
  moe_status st = check_layer_args(d, w);
  if (st != MOE_OK) return st;
  if (n_tokens < 0) return MOE_EINVAL;
  if (n_tokens == 0) return MOE_OK;
  const size_t need = moe_workspace_bytes(d, n_tokens);
  if (need > kNoAllocScratchBytes) return MOE_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (noalloc_scratch(s, &ws) != hipSuccess || !ws) return MOE_EHIP;
  return moe_layer_forward_ex(d, w, x, n_tokens, out, topk_idx_out, topk_w_out, ws, need, stream,
                              nullptr);
}

moe_status moe_rmsnorm(const float* x, int32_t n_tokens, int32_t hidden, float eps, float* out,
                       void* stream) {
  if (n_tokens < 0 || hidden <= 0 || !(eps >= 0.0f)) return MOE_EINVAL;
  if (n_tokens == 0) return MOE_OK;
  if (!x || !out) return MOE_EINVAL;
  if (launch_rmsnorm(x, out, n_tokens, hidden, eps, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return MOE_EHIP;
  return MOE_OK;
}

moe_status moe_stack_forward(const moe_layer_desc* d, const moe_layer_weights* layers,
                             int32_t n_layers, float* x, int32_t n_tokens, float* y_layers,
                             void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->act_dtype != MOE_F32) return MOE_EINVAL;
  if (n_layers < 0 || n_tokens < 0 || !(d->norm_eps >= 0.0f)) return MOE_EINVAL;
  if (n_layers == 0 || n_tokens == 0) return MOE_OK;
  if (!layers || !x || !ws || !aligned16(x) || !aligned16(ws)) return MOE_EINVAL;
  if (y_layers && !aligned16(y_layers)) return MOE_EINVAL;
  for (int l = 0; l < n_layers; ++l) {
    st = check_layer_args(d, &layers[l]);
    if (st != MOE_OK) return st;
  }
  if (ws_bytes < moe_workspace_bytes(d, n_tokens)) return MOE_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Carve c = carve(*d, n_tokens);
  float* xn = at<float>(ws, c.xn);
  const int64_t TH = (int64_t)n_tokens * d->hidden;
  for (int l = 0; l < n_layers; ++l) {
    if (launch_rmsnorm(x, xn, n_tokens, d->hidden, d->norm_eps, s) != hipSuccess) return MOE_EHIP;
    float* ycopy = y_layers ? y_layers + (int64_t)l * TH : nullptr;
    st = layer_impl(*d, layers[l], xn, n_tokens, x, nullptr, nullptr, ws, x, ycopy, s, nullptr);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status moe_dequant_rows(int32_t dtype, const void* codes, const float* scales, int32_t cols,
                            int32_t row0, int32_t n_rows, float* out_f32,
                            uint16_t* out_bf16_codes, void* stream) {
  if (!dtype_is_weight(dtype)) return MOE_EINVAL;
  if (cols <= 0 || row0 < 0 || n_rows < 0) return MOE_EINVAL;
  if (n_rows == 0) return MOE_OK;
  if (!codes || !out_f32) return MOE_EINVAL;
  if (dtype != MOE_BF16 && !scales) return MOE_EINVAL;
  if ((dtype == MOE_I4 && cols % 2) || (dtype == MOE_I2 && cols % 4)) return MOE_EUNSUPPORTED;
  if (dtype == MOE_BF16 && out_bf16_codes) return MOE_EINVAL;
  if (launch_dequant(dtype, codes, scales, cols, row0, n_rows, out_f32, out_bf16_codes,
                     static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_EHIP;
  return MOE_OK;
}

moe_status moe_requant_fp8_int4(const uint8_t* fp8, const float* block_scales, int32_t rows,
                                int32_t cols, int32_t block, uint8_t* codes, float* scales,
                                void* stream) {
  if (rows < 0 || cols <= 0 || block <= 0) return MOE_EINVAL;
  if (rows == 0) return MOE_OK;
  if (!fp8 || !block_scales || !codes || !scales) return MOE_EINVAL;
  if (!requant_supported(cols, block)) return MOE_EUNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(fp8) & 7) || (reinterpret_cast<uintptr_t>(codes) & 3))
    return MOE_EINVAL;
  if (launch_requant_fp8_int4(fp8, block_scales, rows, cols, block, codes, scales,
                              static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_EHIP;
  return MOE_OK;
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: shape or type outside the kernels' coverage";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP launch or runtime error";
  }
  return "unknown moe_status";
}

}  // extern "C"
