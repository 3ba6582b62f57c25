// Plain bf16 matrix products through hipBLASLt.
//
// Used where a step of the path is a dense product with no fusion around it
// (the expansion of cached latent rows into per-head keys and values for
// prefill: "MLA, dim by dim", "MLA Prefill").  Column-major convention:
//   C (M x N, ldc) = op(A) (M x K) * op(B) (K x N),
// bf16 inputs and output, fp32 accumulation, alpha = 1, beta = 0, optionally
// batched with element strides between consecutive operands.  The matmul
// descriptor, layouts and the heuristic's algorithm are built once per device
// and shape and kept for the life of the process; no workspace is used.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "mla_internal.h"

namespace mla {

namespace {

constexpr int MAX_DEVICES = 64;

struct GemmPlan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
  hipblasLtMatmulAlgo_t algo;
};

using GemmKey =
    std::tuple<int, int, int, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int, int64_t, int64_t, int64_t>;

std::mutex g_mu;
hipblasLtHandle_t g_handle[MAX_DEVICES] = {};
std::map<GemmKey, GemmPlan> g_plans;

bool set_batch(hipblasLtMatrixLayout_t l, int batch, int64_t stride) {
  if (batch <= 1) return true;
  const int32_t n = batch;
  return hipblasLtMatrixLayoutSetAttribute(l, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &n, sizeof(n)) ==
             HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatrixLayoutSetAttribute(l, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &stride,
                                           sizeof(stride)) == HIPBLAS_STATUS_SUCCESS;
}

bool build_plan(hipblasLtHandle_t h, bool trans_a, bool trans_b, int64_t M, int64_t N, int64_t K, int64_t lda,
                int64_t ldb, int64_t ldc, int batch, int64_t stride_a, int64_t stride_b, int64_t stride_c,
                GemmPlan* plan) {
  if (hipblasLtMatmulDescCreate(&plan->desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return false;
  const int32_t op_a = trans_a ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  const int32_t op_b = trans_b ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  if (hipblasLtMatmulDescSetAttribute(plan->desc, HIPBLASLT_MATMUL_DESC_TRANSA, &op_a, sizeof(op_a)) !=
          HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(plan->desc, HIPBLASLT_MATMUL_DESC_TRANSB, &op_b, sizeof(op_b)) !=
          HIPBLAS_STATUS_SUCCESS)
    return false;
  // stored shapes: op(A) is M x K, so A is K x M when transposed
  if (hipblasLtMatrixLayoutCreate(&plan->a, HIP_R_16BF, trans_a ? K : M, trans_a ? M : K, lda) !=
          HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&plan->b, HIP_R_16BF, trans_b ? N : K, trans_b ? K : N, ldb) !=
          HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&plan->c, HIP_R_16BF, M, N, ldc) != HIPBLAS_STATUS_SUCCESS)
    return false;
  if (!set_batch(plan->a, batch, stride_a) || !set_batch(plan->b, batch, stride_b) ||
      !set_batch(plan->c, batch, stride_c))
    return false;
  hipblasLtMatmulPreference_t pref = nullptr;
  if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return false;
  const uint64_t no_ws = 0;
  hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &no_ws, sizeof(no_ws));
  hipblasLtMatmulHeuristicResult_t res[1];
  int returned = 0;
  const hipblasStatus_t s =
      hipblasLtMatmulAlgoGetHeuristic(h, plan->desc, plan->a, plan->b, plan->c, plan->c, pref, 1, res, &returned);
  hipblasLtMatmulPreferenceDestroy(pref);
  if (s != HIPBLAS_STATUS_SUCCESS || returned < 1 || res[0].state != HIPBLAS_STATUS_SUCCESS) return false;
  plan->algo = res[0].algo;
  return true;
}

}  // namespace

hipError_t gemm_bf16(bool trans_a, bool trans_b, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                     const void* B, int64_t ldb, void* C, int64_t ldc, int batch, int64_t stride_a,
                     int64_t stride_b, int64_t stride_c, hipStream_t stream) {
  if (M <= 0 || N <= 0 || K <= 0 || batch <= 0) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  hipblasLtHandle_t h;
  const GemmPlan* plan;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_handle[dev] == nullptr && hipblasLtCreate(&g_handle[dev]) != HIPBLAS_STATUS_SUCCESS) {
      g_handle[dev] = nullptr;
      return hipErrorNotInitialized;
    }
    h = g_handle[dev];
    const GemmKey key{dev, trans_a, trans_b, M, N, K, lda, ldb, ldc, batch, stride_a, stride_b, stride_c};
    auto it = g_plans.find(key);
    if (it == g_plans.end()) {
      GemmPlan p;
      if (!build_plan(h, trans_a, trans_b, M, N, K, lda, ldb, ldc, batch, stride_a, stride_b, stride_c, &p))
        return hipErrorNotSupported;
      it = g_plans.emplace(key, p).first;
    }
    plan = &it->second;   // map nodes stay put
  }
  const float alpha = 1.0f, beta = 0.0f;
  const hipblasStatus_t s = hipblasLtMatmul(h, plan->desc, &alpha, A, plan->a, B, plan->b, &beta, C, plan->c, C,
                                            plan->c, &plan->algo, nullptr, 0, stream);
  return s == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace mla
