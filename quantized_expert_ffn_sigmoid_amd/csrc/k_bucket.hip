// k_bucket.hip -- batch-union grouping on gfx950 ("colibri" README, "What's
// implemented": each unique expert of the batch is read once and applied to
// every position routed to it).
//
// One workgroup of 1024 threads performs a stable counting sort of the flat
// slots f = t*k + j by expert: an LDS histogram, an exclusive scan, then a
// scatter in rounds of 1024 slots.  Within a round, a slot's rank among equal
// experts is found without atomics: ten ballots over the expert id's bits give
// each lane the mask of lanes in its wave with the same expert; per-wave counts
// in LDS give the offset of earlier waves.  The result is deterministic and
// equals a stable sort.
#include "moe_internal.h"

namespace moe {

constexpr int BK_THREADS = 1024;
constexpr int BK_WAVES = BK_THREADS / kWave;
constexpr int BK_KEY_BITS = 10;   // experts < 1024

__global__ __launch_bounds__(BK_THREADS) void k_bucket(int32_t T, int32_t K, int32_t E,
                                                       const int32_t* __restrict__ idx,
                                                       int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ entries,
                                                       int32_t* __restrict__ inverse,
                                                       int32_t* __restrict__ active,
                                                       int32_t* __restrict__ n_active) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_wcnt[BK_WAVES][kMaxExperts];
  __shared__ int s_scan[BK_THREADS];
  __shared__ int s_flag[BK_THREADS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t F = (int64_t)T * K;

  for (int e = tid; e < E; e += BK_THREADS) {
    s_cnt[e] = 0;
    for (int w = 0; w < BK_WAVES; ++w) s_wcnt[w][e] = 0;
  }
  __syncthreads();
  for (int64_t f = tid; f < F; f += BK_THREADS) {
    const int e = idx[f];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();

  // exclusive scans of the counts and of the nonzero flags (E <= 1024 = one
  // element per thread), Hillis-Steele in LDS
  const int v = tid < E ? s_cnt[tid] : 0;
  const int fl = v > 0 ? 1 : 0;
  s_scan[tid] = v;
  s_flag[tid] = fl;
  __syncthreads();
  for (int d = 1; d < BK_THREADS; d <<= 1) {
    const int a = tid >= d ? s_scan[tid - d] : 0;
    const int b = tid >= d ? s_flag[tid - d] : 0;
    __syncthreads();
    s_scan[tid] += a;
    s_flag[tid] += b;
    __syncthreads();
  }
  if (tid < E) {
    const int excl = s_scan[tid] - v;
    counts[tid] = v;
    offsets[tid] = excl;
    s_base[tid] = excl;
    if (fl) active[s_flag[tid] - 1] = tid;
  }
  if (tid == 0) {
    offsets[E] = s_scan[E - 1];
    n_active[0] = s_flag[E - 1];
  }
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t r0 = 0; r0 < F; r0 += BK_THREADS) {
    const int64_t f = r0 + tid;
    const int e = f < F ? idx[f] : -1;
    const bool valid = e >= 0 && e < E;
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < BK_KEY_BITS; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t bm = __ballot(bit);
      m &= bit ? bm : ~bm;
    }
    const int rank = __popcll(m & lt_mask);
    const int cnt = __popcll(m);
    const bool leader = valid && rank == 0;
    if (leader) s_wcnt[wave][e] = cnt;
    __syncthreads();
    if (valid) {
      int pos = s_base[e] + rank;
      for (int w = 0; w < wave; ++w) pos += s_wcnt[w][e];
      entries[pos] = (int32_t)f;
      inverse[f] = pos;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&s_base[e], cnt);
      s_wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

hipError_t launch_bucket(int32_t T, int32_t K, int32_t E, const int32_t* topk_idx,
                         int32_t* counts, int32_t* offsets, int32_t* entries, int32_t* inverse,
                         int32_t* active, int32_t* n_active, hipStream_t s) {
  hipLaunchKernelGGL(k_bucket, dim3(1), dim3(BK_THREADS), 0, s, T, K, E, topk_idx, counts,
                     offsets, entries, inverse, active, n_active);
  return hipGetLastError();
}

}  // namespace moe
