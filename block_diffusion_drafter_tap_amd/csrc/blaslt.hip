// Plain bf16 GEMMs through hipBLASLt: Y[M][N] = X[M][K] . W[N][K]^T with X and W
// bf16 row-major (leading dimensions ldx and K), Y bf16 or fp32 row-major
// (leading dimension ldo), fp32 accumulation. Used for the staging stage's fc
// projection of a whole context window (4096 rows at the qwen3-4b shape) and for
// its context K/V projections (fp32 rows, whose head epilogue then runs as a
// kernel of its own): dense MFMA-bound products where the library's tuned
// kernels run faster than the tile GEMM of prefill.hip.
//
// In hipBLASLt's column-major terms Y^T (N x M, ld ldo) = op(A) op(B) with A the
// weights as a K x N matrix (ld K, transposed) and B the rows as a K x M matrix
// (ld ldx). One handle per device, created by blaslt_prepare (from the handle
// binding call, never from a stream call), and the descriptors, layouts and the
// heuristic's first algorithm are kept per shape. No workspace is offered, so the
// algorithms chosen need none. When there is no handle for the device, or the
// library offers no algorithm for a shape, the call returns hipErrorNotSupported
// and the caller runs its own kernel instead.
#include <hipblaslt/hipblaslt.h>

#include <mutex>

#include "kernels.h"

namespace {

constexpr int LT_MAX_DEV = 64;
constexpr int LT_MAX_PLANS = 32;

struct LtPlan {
  bool used = false, ok = false;
  int dev, M, N, K, out_f32;
  long long ldx, ldo;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo;
};

std::mutex g_mu;
hipblasLtHandle_t g_handle[LT_MAX_DEV] = {};
bool g_handle_failed[LT_MAX_DEV] = {};
LtPlan g_plans[LT_MAX_PLANS];
int g_next = 0;   // the entry a new shape replaces once all are used

void release(LtPlan& p) {
  if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
  if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
  if (p.lb) hipblasLtMatrixLayoutDestroy(p.lb);
  if (p.lc) hipblasLtMatrixLayoutDestroy(p.lc);
  p = LtPlan();
}

// descriptors, layouts and an algorithm for one shape; p.ok tells whether the
// library has one
void plan(LtPlan& p, hipblasLtHandle_t h) {
  p.ok = false;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, p.K, p.N, p.K) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, p.K, p.M, p.ldx) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.lc, p.out_f32 ? HIP_R_32F : HIP_R_16BF, p.N, p.M, p.ldo) != HIPBLAS_STATUS_SUCCESS)
    return;
  hipblasLtMatmulPreference_t pref = nullptr;
  if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return;
  const uint64_t ws = 0;
  hipblasLtMatmulHeuristicResult_t res[1];
  int n = 0;
  const bool got =
      hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof ws) ==
          HIPBLAS_STATUS_SUCCESS &&
      hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.la, p.lb, p.lc, p.lc, pref, 1, res, &n) == HIPBLAS_STATUS_SUCCESS &&
      n > 0 && res[0].state == HIPBLAS_STATUS_SUCCESS && res[0].workspaceSize == 0;
  hipblasLtMatmulPreferenceDestroy(pref);
  if (!got) return;
  p.algo = res[0].algo;
  p.ok = true;
}

}  // namespace

hipError_t blaslt_prepare() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= LT_MAX_DEV) return hipErrorNotSupported;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_handle[dev]) return hipSuccess;
  if (g_handle_failed[dev]) return hipErrorNotSupported;
  if (hipblasLtCreate(&g_handle[dev]) != HIPBLAS_STATUS_SUCCESS) {
    g_handle[dev] = nullptr;
    g_handle_failed[dev] = true;
    return hipErrorNotSupported;
  }
  return hipSuccess;
}

hipError_t blaslt_gemm_nt(const uint16_t* x, long long ldx, const uint16_t* w, int M, int N, int K, void* out,
                          long long ldo, int out_f32, hipStream_t st) {
  if (!x || !w || !out || M < 1 || N < 1 || K < 1 || ldx < K || ldo < N) return hipErrorInvalidValue;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= LT_MAX_DEV) return hipErrorNotSupported;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_handle[dev]) return hipErrorNotSupported;
  LtPlan* p = nullptr;
  for (auto& q : g_plans)
    if (q.used && q.dev == dev && q.M == M && q.N == N && q.K == K && q.ldx == ldx && q.ldo == ldo &&
        q.out_f32 == out_f32) {
      p = &q;
      break;
    }
  if (!p) {
    p = &g_plans[g_next];
    g_next = (g_next + 1) % LT_MAX_PLANS;
    release(*p);
    p->used = true;
    p->dev = dev;
    p->M = M;
    p->N = N;
    p->K = K;
    p->ldx = ldx;
    p->ldo = ldo;
    p->out_f32 = out_f32;
    plan(*p, g_handle[dev]);
  }
  if (!p->ok) return hipErrorNotSupported;
  const float alpha = 1.0f, beta = 0.0f;
  const hipblasStatus_t s = hipblasLtMatmul(g_handle[dev], p->desc, &alpha, w, p->la, x, p->lb, &beta, out, p->lc, out,
                                            p->lc, &p->algo, nullptr, 0, st);
  return s == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}
