// k_ggemm.hip -- batch-union grouped GEMM on the matrix cores (gfx950), for
// buckets of prefill size.
//
// Each active expert applies its SwiGLU FFN to the rows of its bucket ("colibri"
// README, "What's implemented": batch-union grouping, each unique expert read
// once and applied to every position routed to it; "iliria" README: gate and
// up over one activation, SwiGLU).  With thousands of tokens the buckets hold
// tens to thousands of rows, so the expert contraction is a dense bf16
// matrix product -- the one dense contraction of the layer -- and runs on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//
// Tiles.  A block computes a 64-row tile of one bucket (or of the shared
// expert's token rows) against 256 weight rows: for gate/up, 128 gate rows and
// the 128 up rows paired with them, so SwiGLU is applied in registers; for down,
// 256 output rows.  Each of the 4 waves owns 64 weight rows (four 16-row
// N-subtiles) and all 64 tile rows (four 16-row M-subtiles): 16 accumulator
// tiles.  A tile of at most 32 or 16 valid rows (most buckets of a Zipf-shaped
// routing hold fewer than 64) computes only its first two M-subtiles or its
// first one.  The K dimension advances 128 at a time.
//
// Operands.  Activations (bf16) are staged per K step in LDS, double buffered,
// rows padded to 272 bytes so that the 16-byte operand reads of 16 lanes fall
// on distinct banks.  Weights go straight from HBM to registers: lane l reads
// 16 bytes of weight row (l % 16) for its K group (l / 16), which are exactly
// the operand elements it supplies.  int4 codes become the exact bf16 values
// q + 8 (the offset-binary code), two per packed fp8 -> bf16 conversion; the
// offset, 8 code units, is removed in the epilogue with the row sums of the
// activations (k_rowsum_bf16, one pass over x and one over h).  The pairing
// of the converted codes ((0, 2), (4, 6), (1, 3), (5, 7) of each dword) is
// matched by storing each group of 8 activations in the order
// 0,2,4,6,1,3,5,7.
// bf16 weights need neither step.  Per-row scales commute with the K sum and
// are applied in the epilogue, as in the decode kernels.
#include "moe_internal.h"
#include "unpack.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4g __attribute__((ext_vector_type(4)));

constexpr int GG_BM = 64;          // tile rows (tokens / bucket positions)
constexpr int GG_BK = 128;         // K per step
constexpr int GG_WAVES = 4;
constexpr int GG_THREADS = GG_WAVES * 64;
constexpr int GG_NW = 64;          // weight rows per wave
constexpr float GG_OFF = 8.0f;     // int4 operand = GG_OFF + q

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4g v) { return __builtin_bit_cast(bf16x8, v); }

// int4 codes become the bf16 values q + 8 by i4_to_bf16 (unpack.h); the
// offset of 8 against codes of rms ~4.3 keeps the fp32 accumulation error
// near that of the codes themselves.
//
// Reorder 8 bf16 activations (x0..x7 in 4 dwords) to x0,x2,x4,x6,x1,x3,x5,x7,
// the order of the codes i4_to_bf16 yields.
__device__ __forceinline__ u32x4g perm_0246(u32x4g d) {
  u32x4g r;
  r.x = __builtin_amdgcn_perm(d.y, d.x, 0x05040100u);
  r.y = __builtin_amdgcn_perm(d.w, d.z, 0x05040100u);
  r.z = __builtin_amdgcn_perm(d.y, d.x, 0x07060302u);
  r.w = __builtin_amdgcn_perm(d.w, d.z, 0x07060302u);
  return r;
}

struct GgTile {
  bool shared;
  int e;          // expert (routed)
  int p0;         // first bucket position (routed) or first token (shared)
  int n;          // valid rows
  int nt;         // n-tile index
};

__device__ __forceinline__ bool gg_tile(const GgArgs& a, GgTile& t) {
  // Blocks are dealt to the 8 XCDs round robin (block b runs on XCD b % 8).
  // m-tiles go round robin to the XCDs, so each holds about an eighth of
  // every large expert's tiles and of the small experts, whatever the bucket
  // sizes; an XCD runs all n-tiles of an m-tile back to back, and they share
  // the m-tile's activation rows through its L2.  The weight rows of an
  // expert whose m-tiles sit on several XCDs are read once per XCD.
  const int x = blockIdx.x % 8;
  const int64_t j = blockIdx.x / 8;
  const int64_t rq = (a.max_tiles + 7) / 8;
  if (j < rq * a.nt_r) {
    const int64_t q = j / a.nt_r;
    t.nt = (int)(j - q * a.nt_r);
    const int mt = x + 8 * (int)q;
    // the record is read together with the count (one round trip), from a
    // clamped index that stays inside the tile arrays
    const int mtc = min(mt, a.max_tiles - 1);
    const int used = *a.n_tiles;
    t.e = a.tile_e[mtc];
    t.p0 = a.tile_p0[mtc];
    t.n = a.tile_n[mtc];
    if (mt >= used) return false;
    t.shared = false;
  } else {
    if (a.s_tiles == 0 || a.nt_s == 0) return false;
    const int64_t j2 = j - rq * a.nt_r;
    const int64_t q = j2 / a.nt_s;
    t.nt = (int)(j2 - q * a.nt_s);
    const int mt = x + 8 * (int)q;
    if (mt >= a.s_tiles) return false;
    t.shared = true;
    t.e = 0;
    t.p0 = mt * GG_BM;
    t.n = min(GG_BM, a.T - t.p0);
  }
  return t.n > 0;
}

// Activation stages in LDS: 64 rows x 256 bytes (128 bf16), no padding; the
// 16 pieces of 16 bytes of row r are stored in the order c ^ (r % 16), so the
// operand reads of 16 lanes (16 rows, one piece) fall on 16 distinct bank
// groups.  Two stages: the one the step computes on and the one it fills.
constexpr int GG_XSTAGE = GG_BM * GG_BK * 2;   // 16 KB

// Workgroup barrier after this wave's LDS writes have completed, without the
// release fence of __syncthreads (which would also wait for every global load
// in flight).  The memory clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void gg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The wave's weight rows (N-subtile ns, lane row ln): down, 64 consecutive
// output rows; gate/up, 32 gate rows (ns 0, 1) and the up rows paired with
// them (ns 2, 3), so that SwiGLU is applied in registers.
template <bool DOWN>
__device__ __forceinline__ void gg_weight_rows(const GgTile& t, int rows, int wave, int ln,
                                               int64_t (&wrow)[4]) {
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    if (DOWN) {
      wrow[ns] = (int64_t)t.nt * 256 + wave * GG_NW + ns * 16 + ln;
    } else {
      const int c = t.nt * 128 + wave * 32 + (ns & 1) * 16 + ln;
      wrow[ns] = ns < 2 ? c : rows + c;
    }
  }
}

// Per tile row (thread r < 64): the output row index and, for int4, the
// activation row sum that removes the operand offset.
template <bool I4, bool DOWN>
__device__ __forceinline__ void gg_row_meta(const GgArgs& a, const GgTile& t, int& row, float& rs) {
  row = 0;
  rs = 0.f;
  if (threadIdx.x < GG_BM) {
    const int r = min((int)threadIdx.x, t.n - 1);
    const int pos = t.p0 + r;
    if (DOWN) {
      row = t.shared ? pos : a.entries[pos];
      if (I4) rs = t.shared ? a.rs_hs[pos] : a.rs_h[pos];
    } else {
      row = pos;
      if (I4) rs = a.rs_x[t.shared ? pos : a.entries[pos] / a.top_k];
    }
  }
}

// Epilogue: lane holds rows m = 16 ms + 4 kg + j of column (weight row) ln
// of each N-subtile.  gate/up of int4 experts writes h in the order their
// down projection reads it (0,2,4,6,1,3,5,7 within groups of 8).
template <bool I4, bool DOWN, int MS>
__device__ __forceinline__ void gg_epilogue(const GgArgs& a, const GgTile& t, int rows, int kg,
                                            const f32x4 (&acc)[MS][4], const int64_t (&wrow)[4],
                                            const float (&sc)[4], const int32_t* s_row,
                                            const float* s_rs) {
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = ms * 16 + kg * 4 + j;
      if (m >= t.n) continue;
      const float off = I4 ? GG_OFF * s_rs[m] : 0.f;
      const int64_t orow = s_row[m];
      if constexpr (DOWN) {
        float* yrow = (t.shared ? a.y_s : a.y) + orow * a.H;
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) yrow[wrow[ns]] = sc[ns] * (acc[ms][ns][j] - off);
      } else {
        uint16_t* hrow = (t.shared ? a.h_s : a.h) + orow * rows;
        float* prow = t.shared ? a.hp_s : a.hp;
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
          const float g = sc[ns] * (acc[ms][ns][j] - off);
          const float u = sc[ns + 2] * (acc[ms][ns + 2][j] - off);
          const int64_t c = wrow[ns];
          const int64_t pc = I4 ? (c & ~7) | ((c & 1) ? 4 + ((c & 7) >> 1) : (c & 7) >> 1) : c;
          const float hv = g / (1.0f + expf(-g)) * u;
          hrow[pc] = f32_to_bf16_bits(hv);
          if (prow) prow[orow * rows + c] = hv;
        }
      }
    }
  }
}

// One tile.  WDT: weight format (MOE_I4 or MOE_BF16); DOWN: down projection
// (else gate/up + SwiGLU); GRP: K steps per weight load (int4: 1 or 2; each
// lane then reads 16 * GRP contiguous bytes of each of its rows); NW: K steps
// of weights in flight (two groups); XD: activation register sets in flight;
// GUARD: the step count is not a multiple of the unroll (the last group has
// idle steps); MS: 16-row M-subtiles computed (tiles of at most 16 or 32 valid
// rows skip the matrix instructions, activation staging and LDS reads of the
// rows they do not hold).
//
// Streams.  All global loads go to registers, so the compiler tracks each of
// them and waits for exactly the ones an instruction needs (vector memory
// completes in issue order).  Activations: the block loads step kt + 1 + XD
// into the register set freed by writing step kt + 1 to the LDS stage that
// step kt + 1 computes on, so each activation tile has XD steps to arrive.
// Weights: the group of step kt + NW is loaded into the registers the group
// of step kt has just consumed.
//
// Groups: the K order inside a group follows the loads: step s of group q
// takes, for lane group kg, the codes q * 128 GRP + kg * 32 GRP + 32 s +
// [0, 32), and the activation stages gather the same positions.
template <int WDT, bool DOWN, int GRP, int NW, int XD, bool GUARD, int MS>
__device__ __forceinline__ void gg_run(const GgArgs& a, const GgTile& t, uint8_t* lds) {
  constexpr bool I4 = WDT == MOE_I4;
  static_assert(I4 || GRP == 1, "bf16 weights load one step at a time");
  static_assert(NW % GRP == 0, "whole groups in flight");
  constexpr int U = NW > XD ? NW : XD;   // unroll: whole register rotations
  static_assert(U % NW == 0 && U % XD == 0, "unroll covers both rotations");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, kg = lane >> 4;
  const ExpertSetDev& ws = t.shared ? a.ws : a.w;
  const int K = DOWN ? (t.shared ? a.Is : a.I) : a.H;
  const int rows = DOWN ? a.H : (t.shared ? a.Is : a.I);   // gate/up: rows of each half
  const uint8_t* W = DOWN ? ws.dn + (int64_t)t.e * ws.dn_stride : ws.gu + (int64_t)t.e * ws.gu_stride;
  const float* S = reinterpret_cast<const float*>(DOWN ? ws.dns + (int64_t)t.e * ws.dns_stride
                                                        : ws.gus + (int64_t)t.e * ws.gus_stride);
  const int64_t rowb = I4 ? K / 2 : (int64_t)K * 2;

  int64_t wrow[4];
  gg_weight_rows<DOWN>(t, rows, wave, ln, wrow);
  const uint8_t* wp[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) wp[ns] = W + wrow[ns] * rowb;

  // Per-tile row data for the epilogue, loaded first so that its latency
  // overlaps the K loop: the lane's four weight-row scales (registers), and
  // per tile row the output row index and, for int4, the activation row sum
  // (LDS, published by the first barrier of the K loop).
  float sc[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) sc[ns] = I4 ? S[wrow[ns]] : 1.0f;
  int32_t* s_row = reinterpret_cast<int32_t*>(lds + 2 * GG_XSTAGE);
  float* s_rs = reinterpret_cast<float*>(s_row + GG_BM);
  int meta_row;
  float meta_rs;
  gg_row_meta<I4, DOWN>(a, t, meta_row, meta_rs);

  // Activation loads: thread (rb = tid / 16, p = tid % 16) moves stored
  // position p of tile rows rb + 16 i (i < 4), which holds logical piece
  // p ^ rb.  int4 weights yield their codes in the order 0,2,4,6,1,3,5,7 of
  // each group of 8, so their activations are read from rows stored in that
  // order (x_p, and h as gate/up writes it).
  const int xp = threadIdx.x & 15, xrb = threadIdx.x >> 4;
  const int xc = xp ^ xrb;   // logical piece
  // the rows' sources: for routed gate/up tiles the bucket entries, read
  // before the first weights so that the two latencies overlap
  int src[MS];
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int pos = t.p0 + min(xrb + 16 * i, t.n - 1);
    src[i] = (DOWN || t.shared) ? pos : a.entries[pos];
  }
  const uint8_t* xsrc[MS];
  auto make_xsrc = [&]() {
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      const uint16_t* row;
      if (DOWN) row = (t.shared ? a.h_s : a.h) + (int64_t)src[i] * K;
      else row = (I4 ? a.x_p : a.x) + (int64_t)(t.shared ? src[i] : src[i] / a.top_k) * K;
      xsrc[i] = reinterpret_cast<const uint8_t*>(row) + (xc >> 2) * (64 * GRP) + (xc & 3) * 16;
    }
  };
  const int nk = K / GG_BK;
  auto load_x = [&](int kt, u32x4g (&v)[MS]) {
    const int64_t off = (int64_t)(kt / GRP) * (256 * GRP) + (kt % GRP) * 64;
#pragma unroll
    for (int i = 0; i < MS; ++i) v[i] = *reinterpret_cast<const u32x4g*>(xsrc[i] + off);
  };
  auto store_x = [&](int buf, const u32x4g (&v)[MS]) {
#pragma unroll
    for (int i = 0; i < MS; ++i)
      *reinterpret_cast<u32x4g*>(lds + buf * GG_XSTAGE + (xrb + 16 * i) * (GG_BK * 2) + xp * 16) = v[i];
  };
  // weights: per group and N-subtile, int4 16 * GRP bytes, bf16 64 bytes
  constexpr int WV = I4 ? GRP : 4;
  auto load_w = [&](int kt, u32x4g (&v)[4][WV]) {
#pragma unroll
    for (int ns = 0; ns < 4; ++ns)
#pragma unroll
      for (int i = 0; i < WV; ++i) {
        const int64_t off = I4 ? (int64_t)(kt / GRP) * (64 * GRP) + kg * (16 * GRP) + i * 16
                               : (int64_t)kt * 256 + kg * 64 + i * 16;
        // ordinary (cached) loads: the m-tiles of an expert re-read these
        // rows and find them in L2
        v[ns][i] = *reinterpret_cast<const u32x4g*>(wp[ns] + off);
      }
  };

  f32x4 acc[MS][4];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: the first NW weight steps, activation sets of steps 0 ..
  // XD - 1, step 0 into stage 0 and its register set refilled with step XD
  constexpr int NWB = NW / GRP;   // weight register groups
  // (the weights first: they do not wait for the bucket entries)
  u32x4g xr[XD][MS];
  u32x4g wbuf[NWB][4][WV];
#pragma unroll
  for (int st = 0; st < NW; ++st)
    if (st % GRP == GRP - 1) load_w(min(st, nk - 1), wbuf[st / GRP]);
  make_xsrc();
#pragma unroll
  for (int j = 0; j < XD; ++j) load_x(min(j, nk - 1), xr[j]);
  store_x(0, xr[0]);
  load_x(min(XD, nk - 1), xr[0]);
  if (threadIdx.x < GG_BM) {
    s_row[threadIdx.x] = meta_row;
    s_rs[threadIdx.x] = meta_rs;
  }

  // The loop is unrolled by U so that every register set has a fixed name;
  // all loads are unconditional (steps past the end repeat the last one) and,
  // without GUARD, the body has no branches.
  for (int kt0 = 0; kt0 < nk; kt0 += U) {
#pragma unroll
    for (int st = 0; st < U; ++st) {
      const int kt = kt0 + st;
      // stage kt & 1 is complete, and every wave is done with stage
      // (kt + 1) & 1, which step kt - 1 computed on
      gg_barrier();
      store_x((kt + 1) & 1, xr[(st + 1) % XD]);
      load_x(min(kt + 1 + XD, nk - 1), xr[(st + 1) % XD]);
      const uint8_t* xs = lds + (kt & 1) * GG_XSTAGE;
      // pin this step's weights here: without it the compiler hoists the
      // conversions of all stages to the top of the group, waiting there for
      // every load in flight
      const int wsl = (st / GRP) % NWB;   // weight group of this step
#pragma unroll
      for (int ns = 0; ns < 4; ++ns)
#pragma unroll
        for (int i = 0; i < WV; ++i) {
          if (!I4 || i == st % GRP) asm volatile("" : "+v"(wbuf[wsl][ns][i]));
        }
      if (!GUARD || kt < nk) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          bf16x8 av[MS];
#pragma unroll
          for (int ms = 0; ms < MS; ++ms)
            av[ms] = as_bf16x8(*reinterpret_cast<const u32x4g*>(
                xs + (16 * ms + ln) * (GG_BK * 2) + 16 * ((kg * 4 + d) ^ ln)));
#pragma unroll
          for (int ns = 0; ns < 4; ++ns) {
            bf16x8 bv;
            if constexpr (I4) {
              const u32x4g wq = wbuf[wsl][ns][st % GRP];
              const uint32_t w = d == 0 ? wq.x : d == 1 ? wq.y : d == 2 ? wq.z : wq.w;
              bv = as_bf16x8(i4_to_bf16(w));
            } else {
              bv = as_bf16x8(wbuf[wsl][ns][d]);
            }
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
              acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[ms], bv, acc[ms][ns], 0, 0, 0);
          }
        }
      }
      // weight refill: the group of step kt + NW into the registers consumed
      if (st % GRP == GRP - 1) load_w(min(kt + NW, nk - 1), wbuf[wsl]);
    }
  }

  gg_epilogue<I4, DOWN, MS>(a, t, rows, kg, acc, wrow, sc, s_row, s_rs);
}

// Waits until at most N vector memory loads of this wave are outstanding.
// The asm form keeps memory accesses from moving across the wait; the
// builtin repeats it in a form the compiler's own wait insertion sees.
// The counts assume that the only vector memory instructions in flight are
// the pipeline's own loads; the built code holds no register spills (scratch
// accesses) between a tile's first direct load and its final wait.
template <int N>
__device__ __forceinline__ void gg_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  // gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt at their
  // maxima (no wait)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) void* gg_lds_ptr;

// Activation stages of the direct-load tile: D + 1 of them, each MS * 16 rows
// of 256 bytes laid out as in GG_XSTAGE.
constexpr int GG_LDS_D = 3;
constexpr int GG_LDS_DIRECT = (GG_LDS_D + 1) * GG_XSTAGE;

// One int4 tile whose activations go from memory straight into the LDS
// stages (global_load_lds), D steps ahead of the step that reads them, and
// whose weights go to registers D steps ahead too, one K step (16 bytes of
// each of the lane's four rows) per load.  Against the register-staged tile
// (gg_run) this frees the activation registers and, with both streams the
// same distance ahead, a wait for one step's activations never holds back on
// a later step's weights: loads complete in issue order, and every load
// issued before a step's activations is needed by that step or an earlier
// one.  At the start of step kt the loads of steps kt + 1 .. kt + D - 1 (MS
// activation loads and 4 weight loads each) may still be in flight; the
// barrier after the wait publishes every wave's activation stage and frees
// the stage of step kt - 1, which the block refills with step kt + D.
// Steps past the end reload the last one (every wave issues the same loads,
// so the counts hold to the end).  K order within a step is that of gg_run
// with GRP = 1.
template <bool DOWN, int MS, int D>
__device__ __forceinline__ void gg_run_lds(const GgArgs& a, const GgTile& t, uint8_t* lds) {
  constexpr int S = D + 1;
  static_assert(S * GG_XSTAGE <= GG_LDS_DIRECT, "stages fit the block's LDS");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = lane & 15, kg = lane >> 4;
  const ExpertSetDev& ws = t.shared ? a.ws : a.w;
  const int K = DOWN ? (t.shared ? a.Is : a.I) : a.H;
  const int rows = DOWN ? a.H : (t.shared ? a.Is : a.I);
  const uint8_t* W = DOWN ? ws.dn + (int64_t)t.e * ws.dn_stride : ws.gu + (int64_t)t.e * ws.gu_stride;
  const float* Sc = reinterpret_cast<const float*>(DOWN ? ws.dns + (int64_t)t.e * ws.dns_stride
                                                         : ws.gus + (int64_t)t.e * ws.gus_stride);
  const int64_t rowb = K / 2;
  int64_t wrow[4];
  gg_weight_rows<DOWN>(t, rows, wave, ln, wrow);
  const uint8_t* wp[4];
  float sc[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    wp[ns] = W + wrow[ns] * rowb + kg * 16;
    sc[ns] = Sc[wrow[ns]];
  }
  int32_t* s_row = reinterpret_cast<int32_t*>(lds + GG_LDS_DIRECT);
  float* s_rs = reinterpret_cast<float*>(s_row + GG_BM);
  int meta_row;
  float meta_rs;
  gg_row_meta<true, DOWN>(a, t, meta_row, meta_rs);

  // Activation loads: one instruction of wave w fills 1 KB of a stage, rows
  // 4w + 16i .. 4w + 16i + 3; lane l takes row 4w + 16i + (l >> 4), stored
  // position l & 15, which holds logical piece (l & 15) ^ (row % 16).
  const int xp = lane & 15, xr = 4 * wave + (lane >> 4);
  const int xc = xp ^ xr;
  // the rows' sources: for routed gate/up tiles the bucket entries, read
  // before the first weights so that the two latencies overlap
  int src[MS];
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const int pos = t.p0 + min(xr + 16 * i, t.n - 1);
    src[i] = (DOWN || t.shared) ? pos : a.entries[pos];
  }
  const int nk = K / GG_BK;
  auto issue_x = [&](int kt, int stage, const uint8_t* const (&xsrc)[MS]) {
#pragma unroll
    for (int i = 0; i < MS; ++i)
      __builtin_amdgcn_global_load_lds(xsrc[i] + (int64_t)kt * (GG_BK * 2),
                                       (gg_lds_ptr)(lds + stage * GG_XSTAGE + (4 * wave + 16 * i) * (GG_BK * 2)),
                                       16, 0, 0);
  };
  u32x4g wbuf[S][4];
  auto issue_w = [&](int kt, u32x4g (&v)[4]) {
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) v[ns] = *reinterpret_cast<const u32x4g*>(wp[ns] + (int64_t)kt * 64);
  };
  // The first step's weights, then the activation rows' addresses (a wait
  // for the entries only), then the first step's activations and the next
  // steps' activations and weights: loads complete in issue order, and from
  // x(0) on the sequence is the loop's, x(j) then w(j) (the first step's
  // weights only come earlier), so every step's wait has the same count.
  issue_w(0, wbuf[0]);
  const uint8_t* xsrc[MS];
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    const uint16_t* row;
    if (DOWN) row = (t.shared ? a.h_s : a.h) + (int64_t)src[i] * K;
    else row = a.x_p + (int64_t)(t.shared ? src[i] : src[i] / a.top_k) * K;
    xsrc[i] = reinterpret_cast<const uint8_t*>(row) + xc * 16;
  }

  f32x4 acc[MS][4];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = f32x4{0.f, 0.f, 0.f, 0.f};
  issue_x(0, 0, xsrc);
#pragma unroll
  for (int j = 1; j < D; ++j) {
    issue_x(min(j, nk - 1), j, xsrc);
    issue_w(min(j, nk - 1), wbuf[j]);
  }
  if (threadIdx.x < GG_BM) {
    s_row[threadIdx.x] = meta_row;
    s_rs[threadIdx.x] = meta_rs;
  }
  // unrolled by S so that stages and register sets have fixed names
  for (int kt0 = 0; kt0 < nk; kt0 += S) {
#pragma unroll
    for (int st = 0; st < S; ++st) {
      const int kt = kt0 + st;
      gg_wait_vm<(D - 1) * (MS + 4)>();
      gg_barrier();
      issue_x(min(kt + D, nk - 1), (st + D) % S, xsrc);
      issue_w(min(kt + D, nk - 1), wbuf[(st + D) % S]);
      if (kt < nk) {
        const uint8_t* xs = lds + st * GG_XSTAGE;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          bf16x8 av[MS];
#pragma unroll
          for (int ms = 0; ms < MS; ++ms)
            av[ms] = as_bf16x8(*reinterpret_cast<const u32x4g*>(
                xs + (16 * ms + ln) * (GG_BK * 2) + 16 * ((kg * 4 + d) ^ ln)));
#pragma unroll
          for (int ns = 0; ns < 4; ++ns) {
            const u32x4g wq = wbuf[st][ns];
            const uint32_t w = d == 0 ? wq.x : d == 1 ? wq.y : d == 2 ? wq.z : wq.w;
            const bf16x8 bv = as_bf16x8(i4_to_bf16(w));
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
              acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[ms], bv, acc[ms][ns], 0, 0, 0);
          }
        }
      }
    }
  }
  // the trailing reloads land before the block's LDS is released
  gg_wait_vm<0>();
  gg_epilogue<true, DOWN, MS>(a, t, rows, kg, acc, wrow, sc, s_row, s_rs);
}

// The M-subtile count of a tile follows its valid rows.
template <int WDT, bool DOWN, int GRP, int NW, int XD, bool GUARD>
__device__ __forceinline__ void gg_run_m(const GgArgs& a, const GgTile& t, uint8_t* lds) {
  if (t.n > 32) gg_run<WDT, DOWN, GRP, NW, XD, GUARD, 4>(a, t, lds);
  else if (t.n > 16) gg_run<WDT, DOWN, GRP, NW, XD, GUARD, 2>(a, t, lds);
  else gg_run<WDT, DOWN, GRP, NW, XD, GUARD, 1>(a, t, lds);
}

// int4 tiles run two waves per SIMD (two blocks per CU), so that one wave's
// int4 unpacking and waits overlap the other's matrix instructions.  Tiles
// of more than 16 rows take the direct-load pipeline, 3 steps ahead; tiles of
// at most 16 rows, whose steps are short and whose time is the weight stream,
// take the register-staged one with weights by pairs of K steps, two pairs
// in flight (64 registers), and two activation sets -- on the grouped GEMM
// of 16384 (token, expert) rows of the 6144 x 2048 layer this split was the
// faster of the two pipelines for each tile size.  bf16 tiles (64 weight
// registers per step) run one wave per SIMD with two weight steps and four
// activation sets in flight.
template <bool DOWN>
__device__ __forceinline__ void gg_dispatch_i4(const GgArgs& a, const GgTile& t, uint8_t* lds) {
  const int K = DOWN ? (t.shared ? a.Is : a.I) : a.H;
  const int nk = K / GG_BK;
  if (nk % 4 == 0 && t.n > 16) {
    if (t.n > 32) gg_run_lds<DOWN, 4, GG_LDS_D>(a, t, lds);
    else gg_run_lds<DOWN, 2, GG_LDS_D>(a, t, lds);
    return;
  }
  if (nk % 2 == 0) {
    if (nk % 4 == 0) gg_run_m<MOE_I4, DOWN, 2, 4, 2, false>(a, t, lds);
    else gg_run_m<MOE_I4, DOWN, 2, 4, 2, true>(a, t, lds);
  } else {
    gg_run_m<MOE_I4, DOWN, 1, 2, 2, true>(a, t, lds);
  }
}

template <bool DOWN>
__device__ __forceinline__ void gg_dispatch_bf16(const GgArgs& a, const GgTile& t, uint8_t* lds) {
  const int K = DOWN ? (t.shared ? a.Is : a.I) : a.H;
  const int nk = K / GG_BK;
  if (nk % 4 == 0) gg_run_m<MOE_BF16, DOWN, 1, 2, 4, false>(a, t, lds);
  else gg_run_m<MOE_BF16, DOWN, 1, 2, 4, true>(a, t, lds);
}

constexpr int GG_LDS = 2 * GG_XSTAGE + 2 * GG_BM * 4;
constexpr int GG_LDS_I4 = (GG_LDS_DIRECT > 2 * GG_XSTAGE ? GG_LDS_DIRECT : 2 * GG_XSTAGE) +
                          2 * GG_BM * 4;

// One launch covers tiles of one weight format: the routed tiles (when
// max_tiles > 0) and the shared expert's (when has_shared).  Two int4 blocks
// (64.5 KB of LDS each) share a CU.
template <bool DOWN>
__global__ __launch_bounds__(GG_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_ggemm_i4(GgArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[GG_LDS_I4];
  GgTile t;
  if (!gg_tile(a, t)) return;
  gg_dispatch_i4<DOWN>(a, t, lds);
}

template <bool DOWN>
__global__ __launch_bounds__(GG_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_ggemm_bf16(GgArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[GG_LDS];
  GgTile t;
  if (!gg_tile(a, t)) return;
  gg_dispatch_bf16<DOWN>(a, t, lds);
}

// Tiles of the buckets: active experts in order, ceil(count / 64) tiles each.
__global__ __launch_bounds__(256) void k_make_tiles(const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ active,
                                                    const int32_t* __restrict__ n_active,
                                                    int32_t* __restrict__ tile_e,
                                                    int32_t* __restrict__ tile_p0,
                                                    int32_t* __restrict__ tile_n,
                                                    int32_t* __restrict__ tile_first,
                                                    int32_t* __restrict__ tile_cnt,
                                                    int32_t* __restrict__ n_tiles) {
  constexpr int PER = kMaxExperts / 256;   // active experts per thread
  __shared__ int32_t scan[kMaxExperts];
  __shared__ int32_t part[256];
  const int na = *n_active;
  const int t = threadIdx.x;
  // tile counts of the thread's run of PER active experts, and their sum
  int cnt[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int s = t * PER + i;
    int c = 0;
    if (s < na) {
      const int e = active[s];
      c = (offsets[e + 1] - offsets[e] + GG_BM - 1) / GG_BM;
    }
    cnt[i] = c;
    sum += c;
  }
  // inclusive scan of the 256 runs' sums (Hillis-Steele in LDS)
  part[t] = sum;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int add = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  int run = part[t] - sum;   // tiles before the thread's run
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    scan[t * PER + i] = run;
    run += cnt[i];
  }
  if (t == 255) *n_tiles = part[255];
  __syncthreads();
  for (int s = threadIdx.x; s < na; s += 256) {
    const int e = active[s];
    const int p = offsets[e], cnt = offsets[e + 1] - p;
    const int ntile = (cnt + GG_BM - 1) / GG_BM;
    for (int i = 0, q = scan[s]; i < ntile; ++i, ++q) {
      tile_e[q] = e;
      tile_p0[q] = p + i * GG_BM;
      tile_n[q] = min(GG_BM, cnt - i * GG_BM);
      tile_first[q] = scan[s];
      tile_cnt[q] = ntile;
    }
  }
}

// Row sums (fp32) of bf16 rows, one wave per row; with perm, also a copy of
// the rows with every group of 8 stored in the order 0,2,4,6,1,3,5,7 (the
// activation order int4 tiles read).
__global__ __launch_bounds__(256) void k_rowsum_bf16(const uint16_t* __restrict__ rows, int32_t n,
                                                     int32_t K, float* __restrict__ out,
                                                     uint16_t* __restrict__ perm) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= n) return;
  const uint16_t* p = rows + r * K;
  float s = 0.f;
  for (int c = lane * 8; c < K; c += 512) {
    const u32x4g v = *reinterpret_cast<const u32x4g*>(p + c);
    if (perm) *reinterpret_cast<u32x4g*>(perm + r * K + c) = perm_0246(v);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) s += __uint_as_float(w[d] << 16) + __uint_as_float(w[d] & 0xFFFF0000u);
  }
  s = wave_sum(s);
  if (lane == 0) out[r] = s;
}

hipError_t launch_rowsum_bf16(const uint16_t* rows, int32_t n, int32_t K, float* out,
                              uint16_t* perm, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rowsum_bf16, dim3((n + 3) / 4), dim3(256), 0, s, rows, n, K, out, perm);
  return hipGetLastError();
}

bool ggemm_supported(const moe_layer_desc& d) {
  const bool fmt = (d.expert_dtype == MOE_I4 || d.expert_dtype == MOE_BF16) &&
                   (d.n_shared == 0 || d.shared_dtype == MOE_I4 || d.shared_dtype == MOE_BF16);
  const int64_t Is = (int64_t)d.inter * (d.n_shared > 0 ? d.n_shared : 1);
  return fmt && d.act_dtype == MOE_BF16 && d.hidden % 256 == 0 && d.inter % 128 == 0 &&
         Is % 128 == 0 && d.n_experts <= kMaxExperts;
}

int32_t ggemm_max_tiles(int32_t T, int32_t K, int32_t E) {
  const int64_t slots = (int64_t)T * K;
  const int64_t tiles = (slots + GG_BM - 1) / GG_BM + (slots < E ? slots : E);
  return (int32_t)tiles;
}

hipError_t launch_make_tiles(const int32_t* offsets, const int32_t* active, const int32_t* n_active,
                             int32_t* tile_e, int32_t* tile_p0, int32_t* tile_n,
                             int32_t* tile_first, int32_t* tile_cnt, int32_t* n_tiles,
                             hipStream_t s) {
  hipLaunchKernelGGL(k_make_tiles, dim3(1), dim3(256), 0, s, offsets, active, n_active, tile_e,
                     tile_p0, tile_n, tile_first, tile_cnt, n_tiles);
  return hipGetLastError();
}

hipError_t launch_ggemm(GgArgs a, bool down, int dtype, int shared_dtype, hipStream_t s) {
  // routed tiles and shared tiles of different formats go to separate
  // launches (the two kernels run at different occupancies)
  const bool split = a.has_shared && shared_dtype != dtype;
  auto go = [&](GgArgs q, int wdt) -> hipError_t {
    q.nt_r = down ? q.H / 256 : q.I / 128;
    q.nt_s = q.has_shared ? (down ? q.H / 256 : q.Is / 128) : 0;
    q.s_tiles = q.has_shared ? (q.T + GG_BM - 1) / GG_BM : 0;
    const int64_t total = (int64_t)q.max_tiles * q.nt_r + (int64_t)q.s_tiles * q.nt_s;
    if (total <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)(8 * (((int64_t)q.max_tiles + 7) / 8 * q.nt_r +
                                            ((int64_t)q.s_tiles + 7) / 8 * q.nt_s));
    if (wdt == MOE_I4) {
      if (down) hipLaunchKernelGGL(k_ggemm_i4<true>, dim3(blocks), dim3(GG_THREADS), 0, s, q);
      else hipLaunchKernelGGL(k_ggemm_i4<false>, dim3(blocks), dim3(GG_THREADS), 0, s, q);
    } else {
      if (down) hipLaunchKernelGGL(k_ggemm_bf16<true>, dim3(blocks), dim3(GG_THREADS), 0, s, q);
      else hipLaunchKernelGGL(k_ggemm_bf16<false>, dim3(blocks), dim3(GG_THREADS), 0, s, q);
    }
    return hipGetLastError();
  };
  if (!split) return go(a, dtype);
  GgArgs r = a;
  r.has_shared = 0;
  hipError_t st = go(r, dtype);
  if (st != hipSuccess) return st;
  GgArgs sh = a;
  sh.max_tiles = 0;   // shared tiles only
  return go(sh, shared_dtype);
}

}  // namespace moe
