// Plain row-major bf16 GEMMs for the projections around Orthros attention
// (x W_Q, x W_K, x W_V and the output projection), on hipBLASLt:
// C[M, N] = A[M, K] Wt[N, K]^T with fp32 accumulation and a bf16 result,
// the weight stored out x in (K contiguous in both operands).
//
// hipBLASLt is column-major; a row-major C = A Wt^T is the column-major
// C^T = Wt A^T: Wt is the first operand, stored [K x N] with leading
// dimension K and transposed, A the second ([K x M], leading dimension K).
// With K contiguous in both operands this is the "TN" form, which runs
// about 11% faster than the untransposed one at the layer's shapes. One
// hipBLASLt handle per device and one plan (descriptors plus the
// heuristic's algorithm) per shape are kept for the life of the process.
#include <hipblaslt/hipblaslt.h>
#include <stdio.h>

#include <map>
#include <mutex>
#include <tuple>

#include "common.h"

namespace orthros {
namespace {

struct Plan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo;
};

std::mutex g_mu;
hipblasLtHandle_t g_handle[64] = {nullptr};
std::map<std::tuple<int, int64_t, int64_t, int64_t, size_t>, Plan> g_plans;

const char *status_name(hipblasStatus_t s) {
  switch (s) {
    case HIPBLAS_STATUS_SUCCESS: return "success";
    case HIPBLAS_STATUS_NOT_INITIALIZED: return "not initialized";
    case HIPBLAS_STATUS_ALLOC_FAILED: return "allocation failed";
    case HIPBLAS_STATUS_INVALID_VALUE: return "invalid value";
    case HIPBLAS_STATUS_ARCH_MISMATCH: return "architecture mismatch";
    case HIPBLAS_STATUS_EXECUTION_FAILED: return "execution failed";
    case HIPBLAS_STATUS_INTERNAL_ERROR: return "internal error";
    case HIPBLAS_STATUS_NOT_SUPPORTED: return "not supported";
    default: return "hipBLASLt error";
  }
}

#define ORTHROS_LT(call, what)                                             \
  do {                                                                     \
    hipblasStatus_t st_ = (call);                                          \
    if (st_ != HIPBLAS_STATUS_SUCCESS) {                                   \
      snprintf(msg, msg_len, "%s: %s", what, status_name(st_));            \
      return -1;                                                           \
    }                                                                      \
  } while (0)

int make_plan(hipblasLtHandle_t h, int64_t M, int64_t N, int64_t K,
              size_t ws_bytes, Plan *p, char *msg, size_t msg_len) {
  ORTHROS_LT(hipblasLtMatmulDescCreate(&p->desc, HIPBLAS_COMPUTE_32F, HIP_R_32F),
             "matmul descriptor");
  const hipblasOperation_t op_a = HIPBLAS_OP_T, op_b = HIPBLAS_OP_N;
  ORTHROS_LT(hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_TRANSA,
                                             &op_a, sizeof(op_a)),
             "transa");
  ORTHROS_LT(hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_TRANSB,
                                             &op_b, sizeof(op_b)),
             "transb");
  ORTHROS_LT(hipblasLtMatrixLayoutCreate(&p->la, HIP_R_16BF, K, N, K), "layout W");
  ORTHROS_LT(hipblasLtMatrixLayoutCreate(&p->lb, HIP_R_16BF, K, M, K), "layout A");
  ORTHROS_LT(hipblasLtMatrixLayoutCreate(&p->lc, HIP_R_16BF, N, M, N), "layout C");
  hipblasLtMatmulPreference_t pref;
  ORTHROS_LT(hipblasLtMatmulPreferenceCreate(&pref), "preference");
  uint64_t wsb = ws_bytes;
  hipblasLtMatmulPreferenceSetAttribute(
      pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof(wsb));
  hipblasLtMatmulHeuristicResult_t res[1];
  int n = 0;
  hipblasStatus_t st = hipblasLtMatmulAlgoGetHeuristic(
      h, p->desc, p->la, p->lb, p->lc, p->lc, pref, 1, res, &n);
  hipblasLtMatmulPreferenceDestroy(pref);
  if (st != HIPBLAS_STATUS_SUCCESS || n < 1) {
    snprintf(msg, msg_len, "no hipBLASLt algorithm for M=%lld N=%lld K=%lld",
             (long long)M, (long long)N, (long long)K);
    return -1;
  }
  p->algo = res[0].algo;
  return 0;
}

}  // namespace

int gemm_bf16(const void *A, const void *Wt, void *C, int64_t M, int64_t N,
              int64_t K, void *ws, size_t ws_bytes, hipStream_t stream,
              char *msg, size_t msg_len) {
  if (M == 0 || N == 0) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    snprintf(msg, msg_len, "no current device");
    return -1;
  }
  const Plan *plan = nullptr;
  hipblasLtHandle_t h;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_handle[dev]) ORTHROS_LT(hipblasLtCreate(&g_handle[dev]), "hipblasLtCreate");
    h = g_handle[dev];
    const auto key = std::make_tuple(dev, M, N, K, ws_bytes);
    auto it = g_plans.find(key);
    if (it == g_plans.end()) {
      Plan p;
      if (make_plan(h, M, N, K, ws_bytes, &p, msg, msg_len)) return -1;
      it = g_plans.emplace(key, p).first;
    }
    plan = &it->second;
  }
  const float one = 1.0f, zero = 0.0f;
  ORTHROS_LT(hipblasLtMatmul(h, plan->desc, &one, Wt, plan->la, A, plan->lb,
                             &zero, C, plan->lc, C, plan->lc, &plan->algo, ws,
                             ws_bytes, stream),
             "hipblasLtMatmul");
  return 0;
}

}  // namespace orthros
