// k_gemv.hip -- geometry and dispatch of the expert GEMV (kernels in
// gemv_impl.h, instantiated per weight format in k_gemv_*.hip).
#include "gemv_impl.h"

namespace moe {

template <int WDT>
static bool geo_for(int32_t K, MatGeo& g) {
  // lanes per row: 64, or fewer for short rows; the lane's K-slice (KSL =
  // K / lpr elements) must be one of the compiled slice lengths
  const int epg = Fmt<WDT>::EPG;
  if (K <= 0 || K % epg) return false;
  const int gran = K / epg;
  int lpr = gran >= 64 ? 64 : gran;
  if (lpr & (lpr - 1)) return false;
  if (gran % lpr) return false;
  const int ksl = K / lpr;
  // (K 6144 -> 96; K 8192 -> 128 for every format; K 7168 -> 112 for bf16
  // only, as 112 codes per lane are not whole 32-code granules of the
  // integer formats)
  const bool ok = WDT == MOE_BF16 ? (ksl == 8 || ksl == 16 || ksl == 32 || ksl == 64 ||
                                     ksl == 96 || ksl == 112 || ksl == 128)
                                  : (ksl == 32 || ksl == 64 || ksl == 96 || ksl == 128);
  if (!ok) return false;
  g.lpr = lpr;
  g.rpp = 64 / lpr;
  g.kc = ksl;   // holds the K-slice length
  return true;
}

bool make_geo(int dtype, int32_t K, MatGeo& g) {
  switch (dtype) {
    case MOE_I4: return geo_for<MOE_I4>(K, g);
    case MOE_I2: return geo_for<MOE_I2>(K, g);
    case MOE_I8: return geo_for<MOE_I8>(K, g);
    case MOE_BF16: return geo_for<MOE_BF16>(K, g);
    default: return false;
  }
}

bool gemv_supported(int dtype, int32_t K) {
  MatGeo g;
  return make_geo(dtype, K, g);
}

bool gemv_ring(int dtype, int32_t K) {
  MatGeo g;
  return (dtype == MOE_I4 || dtype == MOE_I2 || dtype == MOE_I8 || dtype == MOE_BF16) &&
         make_geo(dtype, K, g) &&
         g.lpr == 64;
}

bool gemv_pair_supported(int dtype, int32_t K, int sdtype, int32_t Ks) {
  MatGeo g, gs;
  if (!make_geo(dtype, K, g) || !make_geo(sdtype, Ks, gs)) return false;
  if (g.kc != gs.kc || g.lpr != gs.lpr) return false;
  // shared formats compiled next to each routed format: the same one, or bf16
  return sdtype == dtype || sdtype == MOE_BF16;
}

static int64_t row_bytes_of(int dtype, int K, bool pair) {
  const int64_t bytes_x4 = dtype == MOE_I4 ? 2 : dtype == MOE_I2 ? 1 : dtype == MOE_I8 ? 4 : 8;
  return (int64_t)K * bytes_x4 / 4 * (pair ? 2 : 1);
}

// Rows per block so that each of its waves streams about bytes_per_wave of
// codes; a multiple of the rows one pass of a wave takes (the waves deal the
// passes out round robin, so the last ones may take one pass fewer).
static int rows_per_block(const MatGeo& g, int dtype, int K, int rows, bool pair,
                          int64_t bytes_per_wave) {
  int64_t units = bytes_per_wave * kWaves / (row_bytes_of(dtype, K, pair) * g.rpp);
  if (units < 1) units = 1;
  int64_t rb = units * g.rpp;
  if (rb > kMaxRingRows) rb = kMaxRingRows / g.rpp * g.rpp;
  if (rb > rows) rb = rows;
  return (int)(rb < 1 ? 1 : rb);
}

// Relative time one byte of codes takes on a wave (x16).  An int4 byte holds
// two elements and takes the unpack work; measured on the GLM decode layer
// (int4 routed, bf16 shared), a bf16 byte streams in half the time, and
// blocks sized by this weight finish together.
static int64_t cost_per_byte(int dtype, int act_bf16) {
  (void)act_bf16;
  switch (dtype) {
    case MOE_BF16: return 8;
    default: return 16;
  }
}

// Waves a launch aims for: 256 CUs x 8 resident waves (two 4-wave blocks per
// CU: the ring path's LDS and the register budget allow two), one round.
constexpr int64_t kTargetWaves = 2048;
constexpr int64_t kTargetBlocks = kTargetWaves / kWaves;
constexpr int64_t kMinBytesPerWave = 8 * 1024;

// Fills in the geometry, token mode and block sizes of a launch; returns the
// number of GEMV blocks (0: no work) or -1 when a shape is not covered.
// ntmax: tokens one pass of a block takes (1, or 2 where allowed).
long long plan_gemv(GemvArgs& a, bool down, int dtype, int& shared_dtype, int max_rows_per_slot,
                    bool allow_nt2, int& ntmax, int64_t target_blocks) {
  const int kin = down ? a.I : a.H, kin_s = down ? a.Is : a.H;
  const int rows = down ? a.H : a.I, rows_s = down ? a.H : a.Is;
  if (!make_geo(dtype, kin, a.geo)) return -1;
  if (a.has_shared) {
    if (!make_geo(shared_dtype, kin_s, a.geo_s)) return -1;
    if (a.geo_s.kc != a.geo.kc || a.geo_s.lpr != a.geo.lpr) return -1;
  } else {
    a.geo_s = a.geo;
    shared_dtype = dtype;
  }
  // tokens one pass of the kernel takes (two only on short slices, where the
  // second token's activations fit in registers, and not with the 32-byte
  // int8 granules, whose registers they would crowd out); buckets that may hold more
  // switch the launch to token mode, which splits them over blocks instead of
  // making one block pass over its rows again
  ntmax = (allow_nt2 && a.geo.kc <= 32 && dtype != MOE_I8 && max_rows_per_slot >= 2) ? 2 : 1;
  a.per_token = max_rows_per_slot > ntmax;
  if (a.per_token) {
    a.n_slots = a.n_slots == 0 ? 0 : a.src.routed ? a.n_tok * a.src.top_k : a.src.n_rows;
    a.tok_s = ntmax;
    a.ntg_s = (a.n_tok + ntmax - 1) / ntmax;
  } else {
    a.tok_s = a.n_tok;
    a.ntg_s = 1;
  }
  // work of the launch (routed slots bounded by n_slots), in bytes weighted by
  // the time a byte of each format takes, split evenly over the waves of one
  // resident round; blocks whose rows are rounded up must not spill into a
  // second round, so grow the share until they fit
  const int act_bf16 = 0;
  const int64_t mat = row_bytes_of(dtype, kin, !down) * rows;
  const int64_t mat_s = a.has_shared ? row_bytes_of(shared_dtype, kin_s, !down) * rows_s : 0;
  const int64_t c_r = cost_per_byte(dtype, act_bf16), c_s = cost_per_byte(shared_dtype, act_bf16);
  int64_t per_wave = ((int64_t)a.n_slots * mat * c_r + (int64_t)a.ntg_s * mat_s * c_s) /
                     (target_blocks * kWaves);
  if (per_wave < kMinBytesPerWave * c_r) per_wave = kMinBytesPerWave * c_r;
  int nb_s = 0;
  long long blocks = 0;
  for (int it = 0; it < 64; ++it) {
    a.rb = rows_per_block(a.geo, dtype, kin, rows, !down, per_wave / c_r);
    a.nb = (rows + a.rb - 1) / a.rb;
    a.rb_s = a.has_shared ? rows_per_block(a.geo_s, shared_dtype, kin_s, rows_s, !down, per_wave / c_s) : 1;
    nb_s = a.has_shared ? (rows_s + a.rb_s - 1) / a.rb_s : 0;
    blocks = (long long)a.n_slots * a.nb + (long long)nb_s * a.ntg_s;
    if (blocks <= target_blocks) break;
    per_wave += per_wave / 16 + 1;
  }
  a.nb_s = nb_s;
  if (blocks <= 0 || max_rows_per_slot <= 0) return 0;
  return blocks;
}

hipError_t launch_gemv(GemvArgs a, bool down, int dtype, int shared_dtype, int act_bf16,
                       int max_rows_per_slot, hipStream_t s) {
  int ntmax = 1;
  const long long blocks =
      plan_gemv(a, down, dtype, shared_dtype, max_rows_per_slot, true, ntmax, kTargetBlocks);
  if (blocks < 0) return hipErrorInvalidValue;
  if (blocks == 0) return hipSuccess;
  const unsigned nblk = (unsigned)blocks;
  switch (dtype) {
    case MOE_I4: return (down ? gemv_i4_dn : gemv_i4_gu)(a, shared_dtype, ntmax, act_bf16, nblk, s);
    case MOE_I2: return (down ? gemv_i2_dn : gemv_i2_gu)(a, shared_dtype, ntmax, act_bf16, nblk, s);
    case MOE_I8: return (down ? gemv_i8_dn : gemv_i8_gu)(a, shared_dtype, ntmax, act_bf16, nblk, s);
    case MOE_BF16: return (down ? gemv_bf_dn : gemv_bf_gu)(a, shared_dtype, ntmax, act_bf16, nblk, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv_pre(GemvArgs a, const PreArgs& p, bool down, int shared_dtype,
                           int act_bf16, hipStream_t s) {
  if (!a.has_shared || p.blocks <= 0) return hipErrorInvalidValue;
  a.n_slots = 0;
  int ntmax = 1;
  int sd = shared_dtype;
  // the routing blocks hold resident slots of their own (each block takes the
  // kernel's LDS): the shared blocks are sized so that all of them are
  // resident beside the routing blocks, with at least one per CU
  int64_t target = kTargetBlocks - p.blocks;
  if (target < kTargetBlocks / 2) target = kTargetBlocks / 2;
  const long long blocks = plan_gemv(a, down, shared_dtype, sd, a.n_tok, false, ntmax, target);
  if (blocks < 0 || !(a.geo_s.lpr == 64)) return hipErrorInvalidValue;
  const unsigned nblk = (unsigned)(blocks + p.blocks);
  return (down ? gemv_pre_dn : gemv_pre_gu)(a, p, shared_dtype, act_bf16, nblk, s);
}

bool gemv_pre_supported(const moe_layer_desc& d, int32_t Is) {
  if (d.n_shared <= 0 || d.router != MOE_ROUTER_SIGMOID_NOAUX_TC || d.n_experts > 256) return false;
  const int sd = d.shared_dtype;
  if (sd != MOE_BF16 && sd != MOE_I4 && sd != MOE_I8) return false;
  return gemv_ring(sd, d.hidden) && gemv_ring(sd, Is);
}

}  // namespace moe
