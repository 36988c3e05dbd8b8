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
#include "route_device.h"

namespace moe {

__global__ __launch_bounds__(BK_THREADS) void k_bucket(int32_t T, int32_t K, int32_t E,
                                                       const int32_t* __restrict__ idx,
                                                       int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ entries,
                                                       int32_t* __restrict__ inverse,
                                                       int32_t* __restrict__ active,
                                                       int32_t* __restrict__ n_active) {
  bucket_block(T, K, E, idx, counts, offsets, entries, inverse, active, n_active);
}

__global__ __launch_bounds__(256) void k_bucket_small(int32_t T, int32_t K, int32_t E,
                                                      const int32_t* __restrict__ idx,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ entries,
                                                      int32_t* __restrict__ inverse,
                                                      int32_t* __restrict__ active,
                                                      int32_t* __restrict__ n_active) {
  __shared__ BucketSmallLds L;
  bucket_small(T, K, E, idx, counts, offsets, entries, inverse, active, n_active, L);
}

hipError_t launch_bucket(int32_t T, int32_t K, int32_t E, const int32_t* topk_idx,
                         int32_t* counts, int32_t* offsets, int32_t* entries, int32_t* inverse,
                         int32_t* active, int32_t* n_active, hipStream_t s) {
  if ((int64_t)T * K <= BK_SMALL)
    hipLaunchKernelGGL(k_bucket_small, dim3(1), dim3(256), 0, s, T, K, E, topk_idx, counts,
                       offsets, entries, inverse, active, n_active);
  else
    hipLaunchKernelGGL(k_bucket, dim3(1), dim3(BK_THREADS), 0, s, T, K, E, topk_idx, counts,
                       offsets, entries, inverse, active, n_active);
  return hipGetLastError();
}

}  // namespace moe
