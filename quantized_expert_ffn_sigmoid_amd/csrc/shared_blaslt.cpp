// shared_blaslt.cpp -- the shared expert's dense GEMMs for prefill batches
// through hipBLASLt (gfx950).
//
// The shared expert ("colibri" README, "The idea": a dense part beside the
// routed experts) applies one bf16 SwiGLU FFN to every token: with thousands
// of tokens its gate/up and down are plain dense GEMMs (bf16 inputs, fp32
// accumulation and output), which the platform's GEMM library runs faster
// than the grouped-GEMM tiles built for ragged buckets of int4 experts.  The
// SwiGLU between them is k_swiglu_rows (k_misc.hip).
//
// A handle per device is created on the first call that needs it, never
// while the stream is being captured (the caller then keeps the grouped-GEMM
// tiles for that call); the algorithm of each shape is the first of the
// library's heuristic candidates that needs no workspace, chosen once and
// reused, so every call of a shape runs the same kernel (deterministic).
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "moe_internal.h"

namespace moe {

namespace {

struct Plan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  bool ok = false;
};

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;
std::map<std::tuple<int, int, int, int>, Plan> g_plans;

bool capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone;
}

// The handle of the stream's device (created here when absent and the
// stream is not capturing); null when unavailable.
hipblasLtHandle_t handle_for(hipStream_t s, int& dev) {
  if (hipStreamGetDevice(s, &dev) != hipSuccess) return nullptr;
  auto it = g_handles.find(dev);
  if (it != g_handles.end()) return it->second;
  if (capturing(s)) return nullptr;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  hipblasLtHandle_t h = nullptr;
  const bool made = hipblasLtCreate(&h) == HIPBLAS_STATUS_SUCCESS;
  if (cur != dev) (void)hipSetDevice(cur);
  if (!made) return nullptr;
  g_handles[dev] = h;
  return h;
}

// D[M][N] (row-major fp32) = B[M][K] (row-major bf16) x A[N][K]^T (row-major
// bf16): in the library's column-major terms D^T (N x M) = op(A) x B with A
// read as the K x N matrix it is in memory, transposed.
Plan* plan_for(hipblasLtHandle_t h, int dev, int M, int N, int K, hipStream_t s) {
  const auto key = std::make_tuple(dev, M, N, K);
  auto it = g_plans.find(key);
  if (it != g_plans.end()) return it->second.ok ? &it->second : nullptr;
  if (capturing(s)) return nullptr;
  Plan p;
  bool ok = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) ==
            HIPBLAS_STATUS_SUCCESS;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta,
                                              sizeof(ta)) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb,
                                              sizeof(tb)) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, K, N, K) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, K, M, K) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&p.lc, HIP_R_32F, N, M, N) == HIPBLAS_STATUS_SUCCESS;
  if (ok) {
    hipblasLtMatmulPreference_t pref = nullptr;
    ok = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
    const uint64_t no_ws = 0;
    ok = ok && hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                     &no_ws, sizeof(no_ws)) ==
                   HIPBLAS_STATUS_SUCCESS;
    hipblasLtMatmulHeuristicResult_t res[8];
    int n = 0;
    ok = ok && hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.la, p.lb, p.lc, p.lc, pref, 8, res,
                                               &n) == HIPBLAS_STATUS_SUCCESS;
    bool found = false;
    for (int i = 0; ok && i < n && !found; ++i) {
      if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize == 0) {
        p.algo = res[i].algo;
        found = true;
      }
    }
    ok = ok && found;
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  }
  p.ok = ok;
  auto ins = g_plans.emplace(key, p);
  return ok ? &ins.first->second : nullptr;
}

}  // namespace

bool shared_gemm_ready(hipStream_t s, int M, int N1, int K1, int N2, int K2) {
  std::lock_guard<std::mutex> lk(g_mu);
  int dev = 0;
  hipblasLtHandle_t h = handle_for(s, dev);
  if (!h) return false;
  return plan_for(h, dev, M, N1, K1, s) != nullptr && plan_for(h, dev, M, N2, K2, s) != nullptr;
}

hipError_t shared_gemm(int M, int N, int K, const void* A, const void* B, float* D,
                       hipStream_t s) {
  Plan* p = nullptr;
  hipblasLtHandle_t h = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    int dev = 0;
    h = handle_for(s, dev);
    if (h) p = plan_for(h, dev, M, N, K, s);
  }
  if (!p) return hipErrorNotSupported;
  const float alpha = 1.f, beta = 0.f;
  const hipblasStatus_t st = hipblasLtMatmul(h, p->desc, &alpha, A, p->la, B, p->lb, &beta, D,
                                             p->lc, D, p->lc, &p->algo, nullptr, 0, s);
  return st == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace moe
