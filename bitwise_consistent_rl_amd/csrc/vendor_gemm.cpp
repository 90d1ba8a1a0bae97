// The non-invariant mode's large-M projections through the vendor GEMM (hipBLASLt).
//
// BCI_MODE_FAST exists only to quote what batch invariance costs, so it takes the
// choices a throughput engine takes: the vendor library picks a kernel, tile and
// split from each call's shape (M included), so a row's bits depend on the batch it
// runs in.  It is used for the plain-output projections (QKV, O, down) of calls above
// the split-K range, whose epilogue work (RoPE and the cache write, the residual add)
// then runs in the library's own kernels; the gate_up GEMM keeps the fused SiLU*up
// kernel, which is faster than the vendor GEMM plus a separate pass over its output.
// The invariant mode never calls this file.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cstdint>
#include <vector>

#include "kernels.h"

namespace bci {

struct VendorGemm {
  hipblasLtHandle_t handle = nullptr;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  struct Plan {
    int M, N, K;
    hipblasLtMatrixLayout_t a, b, c;
    hipblasLtMatmulAlgo_t algo;
    size_t ws_need;
  };
  std::vector<Plan> plans;
};

void vendor_gemm_destroy(VendorGemm* v) {
  if (!v) return;
  for (auto& p : v->plans) {
    (void)hipblasLtMatrixLayoutDestroy(p.a);
    (void)hipblasLtMatrixLayoutDestroy(p.b);
    (void)hipblasLtMatrixLayoutDestroy(p.c);
  }
  if (v->pref) (void)hipblasLtMatmulPreferenceDestroy(v->pref);
  if (v->desc) (void)hipblasLtMatmulDescDestroy(v->desc);
  if (v->handle) (void)hipblasLtDestroy(v->handle);
  delete v;
}

bool vendor_gemm_create(VendorGemm** out, void* ws, size_t ws_bytes) {
  *out = nullptr;
  VendorGemm* v = new VendorGemm();
  v->ws = ws;
  v->ws_bytes = ws_bytes;
  // row-major C[M, N] = A[M, K] . W[N, K]^T is, column-major, C^T[N, M] = W^T' . A^T':
  // the library's A is W ([K, N] column-major, transposed), its B is A ([K, M], as is)
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  if (hipblasLtCreate(&v->handle) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescCreate(&v->desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(v->desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta) !=
          HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(v->desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb) !=
          HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulPreferenceCreate(&v->pref) != HIPBLAS_STATUS_SUCCESS) {
    vendor_gemm_destroy(v);
    return false;
  }
  const uint64_t wsb = ws_bytes;
  if (hipblasLtMatmulPreferenceSetAttribute(v->pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb,
                                            sizeof wsb) != HIPBLAS_STATUS_SUCCESS) {
    vendor_gemm_destroy(v);
    return false;
  }
  *out = v;
  return true;
}

// C [M, N] bf16 = A [M, K] . W [N, K]^T, fp32 accumulation.  The first call of a shape
// asks the library's heuristic for an algorithm and keeps it.  Returns false when the
// library has no algorithm for the shape or the launch fails.
bool vendor_gemm(VendorGemm* v, const void* A, const void* W, void* C, int M, int N, int K, hipStream_t s) {
  if (M == 0) return true;
  VendorGemm::Plan* plan = nullptr;
  for (auto& p : v->plans)
    if (p.M == M && p.N == N && p.K == K) plan = &p;
  if (!plan) {
    VendorGemm::Plan p{M, N, K, nullptr, nullptr, nullptr, {}, 0};
    if (hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16BF, K, N, K) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.b, HIP_R_16BF, K, M, K) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.c, HIP_R_16BF, N, M, N) != HIPBLAS_STATUS_SUCCESS)
      return false;
    hipblasLtMatmulHeuristicResult_t res[1];
    int got = 0;
    if (hipblasLtMatmulAlgoGetHeuristic(v->handle, v->desc, p.a, p.b, p.c, p.c, v->pref, 1, res, &got) !=
            HIPBLAS_STATUS_SUCCESS ||
        got < 1 || res[0].workspaceSize > v->ws_bytes) {
      (void)hipblasLtMatrixLayoutDestroy(p.a);
      (void)hipblasLtMatrixLayoutDestroy(p.b);
      (void)hipblasLtMatrixLayoutDestroy(p.c);
      return false;
    }
    p.algo = res[0].algo;
    p.ws_need = res[0].workspaceSize;
    v->plans.push_back(p);
    plan = &v->plans.back();
  }
  const float alpha = 1.0f, beta = 0.0f;
  return hipblasLtMatmul(v->handle, v->desc, &alpha, W, plan->a, A, plan->b, &beta, C, plan->c, C, plan->c,
                         &plan->algo, v->ws, plan->ws_need, s) == HIPBLAS_STATUS_SUCCESS;
}

}  // namespace bci
