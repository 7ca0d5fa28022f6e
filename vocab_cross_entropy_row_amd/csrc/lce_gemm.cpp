// Plain library GEMMs (hipBLASLt) used by the fused projection's backward.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cstdint>
#include <map>
#include <mutex>
#include <tuple>

#include "lce.h"
#include "lce_host.h"

namespace lce {
namespace host {

// ------------------------------------------------------------ library GEMMs
// The two plain products of the fused-projection backward (dx = dZ W and
// dW = dZ^T x) go to hipBLASLt: bf16 operands, fp32 accumulation and output.
// One handle per device and one plan (descriptors, layouts and the heuristic's
// first algorithm) per GEMM shape, created on first use and kept for the
// process's lifetime.
struct GemmPlan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  size_t ws = 0;
};
typedef std::tuple<int, int, int, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, size_t>
    GemmKey;
std::map<int, hipblasLtHandle_t> g_blaslt;
std::map<GemmKey, GemmPlan> g_gemm_plans;
std::mutex g_gemm_mu;

lce_status blas_fail(hipblasStatus_t st, const char* what) {
  return fail(LCE_ERR_HIP, "hipBLASLt %s failed (status %d)", what, (int)st);
}

// D (fp32, column-major m x n, leading dimension ldd) = op(A) op(B) + beta D
// with bf16 A and B (column-major, op N or T).  `ws` is device workspace.
lce_status gemm_bf16_f32(hipblasOperation_t ta, hipblasOperation_t tb, int64_t m, int64_t n,
                         int64_t k, const void* A, int64_t lda, const void* B, int64_t ldb,
                         float beta, float* D, int64_t ldd, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipblasLtHandle_t h = nullptr;
  GemmPlan plan;
  {
    std::lock_guard<std::mutex> lock(g_gemm_mu);
    const GemmKey key{dev, (int)ta, (int)tb, m, n, k, lda, ldb, ldd, ws_bytes};
    auto hit = g_gemm_plans.find(key);
    if (hit != g_gemm_plans.end()) {
      plan = hit->second;
      h = g_blaslt[dev];
    } else {
      // Creating a handle or a plan is not allowed inside a graph capture.
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      e = hipStreamIsCapturing(stream, &cap);
      if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
      if (cap != hipStreamCaptureStatusNone)
        return fail(LCE_ERR_UNSUPPORTED,
                    "stream is being captured and this GEMM shape has not been planned yet: make "
                    "one call of the same shape on this device before capture");
      hipblasStatus_t st = HIPBLAS_STATUS_SUCCESS;
      auto it = g_blaslt.find(dev);
      if (it == g_blaslt.end()) {
        if ((st = hipblasLtCreate(&h)) != HIPBLAS_STATUS_SUCCESS) return blas_fail(st, "handle creation");
        g_blaslt[dev] = h;
      } else {
        h = it->second;
      }
      // On any failure below, what was created so far is released (a plan is
      // kept only once it is complete).
      auto drop = [&plan](lce_status r) {
        if (plan.d) hipblasLtMatrixLayoutDestroy(plan.d);
        if (plan.b) hipblasLtMatrixLayoutDestroy(plan.b);
        if (plan.a) hipblasLtMatrixLayoutDestroy(plan.a);
        if (plan.desc) hipblasLtMatmulDescDestroy(plan.desc);
        return r;
      };
      if ((st = hipblasLtMatmulDescCreate(&plan.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F)) != HIPBLAS_STATUS_SUCCESS)
        return drop(blas_fail(st, "descriptor creation"));
      const int32_t opa = (int32_t)ta, opb = (int32_t)tb;
      hipblasLtMatmulDescSetAttribute(plan.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof opa);
      hipblasLtMatmulDescSetAttribute(plan.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof opb);
      const bool an = ta == HIPBLAS_OP_N, bn = tb == HIPBLAS_OP_N;
      if ((st = hipblasLtMatrixLayoutCreate(&plan.a, HIP_R_16BF, an ? m : k, an ? k : m, lda)) != HIPBLAS_STATUS_SUCCESS ||
          (st = hipblasLtMatrixLayoutCreate(&plan.b, HIP_R_16BF, bn ? k : n, bn ? n : k, ldb)) != HIPBLAS_STATUS_SUCCESS ||
          (st = hipblasLtMatrixLayoutCreate(&plan.d, HIP_R_32F, m, n, ldd)) != HIPBLAS_STATUS_SUCCESS)
        return drop(blas_fail(st, "layout creation"));
      hipblasLtMatmulPreference_t pref = nullptr;
      if ((st = hipblasLtMatmulPreferenceCreate(&pref)) != HIPBLAS_STATUS_SUCCESS)
        return drop(blas_fail(st, "preference creation"));
      const uint64_t wsb = ws_bytes;
      hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof wsb);
      hipblasLtMatmulHeuristicResult_t res[1];
      int found = 0;
      st = hipblasLtMatmulAlgoGetHeuristic(h, plan.desc, plan.a, plan.b, plan.d, plan.d, pref, 1, res, &found);
      hipblasLtMatmulPreferenceDestroy(pref);
      if (st != HIPBLAS_STATUS_SUCCESS || found < 1)
        return drop(fail(LCE_ERR_UNSUPPORTED, "hipBLASLt has no algorithm for a %lld x %lld x %lld GEMM (status %d)",
                         (long long)m, (long long)n, (long long)k, (int)st));
      plan.algo = res[0].algo;
      plan.ws = res[0].workspaceSize;
      g_gemm_plans[key] = plan;
    }
  }
  const float alpha = 1.0f;
  hipblasStatus_t st = hipblasLtMatmul(h, plan.desc, &alpha, A, plan.a, B, plan.b, &beta, D, plan.d,
                                       D, plan.d, &plan.algo, ws, plan.ws, stream);
  if (st != HIPBLAS_STATUS_SUCCESS) return blas_fail(st, "matmul");
  note_launch("hipBLASLt GEMM m %lld n %lld k %lld", (long long)m, (long long)n, (long long)k);
  return LCE_OK;
}

}  // namespace host
}  // namespace lce
