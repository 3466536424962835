// hipBLASLt's MXFP4 GEMM behind a small C ABI, for measurement and
// cross-checking only: the benchmark times it beside fp4mx_gemm on the same
// operands, and a GPU test compares the two outputs element by element.  It
// is built into its own library (libfp4mx_vendor.so); no entry point of
// libfp4mx.so calls it.
//
// Operation and layouts are those of fp4mx_gemm: C[m][n] (fp32, row-major,
// ldc = n) = alpha * A . B^T with A [m][k] and B [n][k] MXFP4 (E2M1 codes two
// per byte, low nibble first, along k; one E8M0 scale byte per 32 elements
// along k, [rows][k/32]).  In hipBLASLt's column-major terms the row-major
// C[m][n] is an n x m matrix D = op(B) . A with op(B) = B^T: our B is
// hipBLASLt's A (stored k x n, transposed), our A its B (stored k x m), and
// both scale tensors hold one byte per 32-element block along k, the
// innermost dimension (HIPBLASLT_MATMUL_MATRIX_SCALE_VEC32_UE8M0).
//
// Functions (all return 0 on success, a negative code on failure):
//   fp4mx_vendor_plan_create(m, n, k, &plan, &nalgos): handle, descriptors,
//     up to 8 heuristic algorithms and a workspace for the largest of them;
//   fp4mx_vendor_gemm(plan, algo, a, as, b, bs, alpha, c, stream): one call of
//     algorithm `algo` (0 .. nalgos-1) on `stream` (hipStream_t, 0 = null);
//   fp4mx_vendor_plan_destroy(plan).
// Plans are created and used by one thread at a time.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>
#include <stdint.h>

#include <new>

namespace {

constexpr int kMaxAlgos = 8;

// One hipBLASLt handle per process, created by the first plan and kept:
// creating a handle loads the library's kernel catalogue.
hipblasLtHandle_t g_handle = nullptr;

struct Plan {
  hipblasLtHandle_t h = nullptr;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulHeuristicResult_t algos[kMaxAlgos];
  int nalgos = 0;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  int64_t m = 0, n = 0, k = 0;
};

void destroy(Plan* p) {
  if (!p) return;
  if (p->ws) (void)hipFree(p->ws);
  if (p->la) hipblasLtMatrixLayoutDestroy(p->la);
  if (p->lb) hipblasLtMatrixLayoutDestroy(p->lb);
  if (p->lc) hipblasLtMatrixLayoutDestroy(p->lc);
  if (p->desc) hipblasLtMatmulDescDestroy(p->desc);
  delete p;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int fp4mx_vendor_plan_create(int64_t m, int64_t n, int64_t k,
                                                                    void** plan, int* nalgos) {
  if (!plan || !nalgos || m <= 0 || n <= 0 || k <= 0 || k % 32 != 0) return -2;
  *plan = nullptr;
  *nalgos = 0;
  Plan* p = new (std::nothrow) Plan();
  if (!p) return -3;
  p->m = m;
  p->n = n;
  p->k = k;
  const hipDataType fp4 = HIP_R_4F_E2M1;
  if (!g_handle && hipblasLtCreate(&g_handle) != HIPBLAS_STATUS_SUCCESS) g_handle = nullptr;
  p->h = g_handle;
  bool ok = p->h != nullptr &&
            hipblasLtMatmulDescCreate(&p->desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
  if (ok) {
    const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    const hipblasLtMatmulMatrixScale_t mode = HIPBLASLT_MATMUL_MATRIX_SCALE_VEC32_UE8M0;
    ok = hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_A_SCALE_MODE, &mode, sizeof(mode)) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_B_SCALE_MODE, &mode, sizeof(mode)) == HIPBLAS_STATUS_SUCCESS;
  }
  // hipBLASLt A = our B (k x n, leading dimension k), B = our A (k x m), D = n x m
  ok = ok && hipblasLtMatrixLayoutCreate(&p->la, fp4, (uint64_t)k, (uint64_t)n, k) == HIPBLAS_STATUS_SUCCESS &&
       hipblasLtMatrixLayoutCreate(&p->lb, fp4, (uint64_t)k, (uint64_t)m, k) == HIPBLAS_STATUS_SUCCESS &&
       hipblasLtMatrixLayoutCreate(&p->lc, HIP_R_32F, (uint64_t)n, (uint64_t)m, n) == HIPBLAS_STATUS_SUCCESS;
  if (ok) {
    // the scale pointers must be set before the heuristic query; any
    // non-null device address serves, the real ones are set per call
    const void* dummy = reinterpret_cast<const void*>(256);
    ok = hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_A_SCALE_POINTER, &dummy, sizeof(dummy)) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_B_SCALE_POINTER, &dummy, sizeof(dummy)) == HIPBLAS_STATUS_SUCCESS;
  }
  if (ok) {
    hipblasLtMatmulPreference_t pref = nullptr;
    const uint64_t max_ws = 256ull << 20;
    ok = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &max_ws, sizeof(max_ws)) == HIPBLAS_STATUS_SUCCESS;
    int got = 0;
    ok = ok && hipblasLtMatmulAlgoGetHeuristic(p->h, p->desc, p->la, p->lb, p->lc, p->lc, pref, kMaxAlgos,
                                               p->algos, &got) == HIPBLAS_STATUS_SUCCESS;
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (ok) {
      for (int i = 0; i < got; ++i)
        if (p->algos[i].state == HIPBLAS_STATUS_SUCCESS) {
          p->algos[p->nalgos++] = p->algos[i];
          if (p->algos[i].workspaceSize > p->ws_bytes) p->ws_bytes = p->algos[i].workspaceSize;
        }
      ok = p->nalgos > 0;
    }
  }
  if (ok && p->ws_bytes > 0) ok = hipMalloc(&p->ws, p->ws_bytes) == hipSuccess;
  if (!ok) {
    destroy(p);
    return -4;
  }
  *plan = p;
  *nalgos = p->nalgos;
  return 0;
}

__attribute__((visibility("default"))) int fp4mx_vendor_gemm(void* plan, int algo, const uint8_t* a,
                                                             const uint8_t* as, const uint8_t* b,
                                                             const uint8_t* bs, float alpha, float* c,
                                                             void* stream) {
  Plan* p = static_cast<Plan*>(plan);
  if (!p || algo < 0 || algo >= p->nalgos || !a || !as || !b || !bs || !c) return -2;
  const void* sa = bs;  // hipBLASLt's A is our B
  const void* sb = as;
  if (hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_A_SCALE_POINTER, &sa, sizeof(sa)) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_B_SCALE_POINTER, &sb, sizeof(sb)) != HIPBLAS_STATUS_SUCCESS)
    return -4;
  const float beta = 0.0f;
  const hipblasStatus_t st =
      hipblasLtMatmul(p->h, p->desc, &alpha, b, p->la, a, p->lb, &beta, c, p->lc, c, p->lc,
                      &p->algos[algo].algo, p->ws, p->ws_bytes, static_cast<hipStream_t>(stream));
  return st == HIPBLAS_STATUS_SUCCESS ? 0 : -5;
}

__attribute__((visibility("default"))) void fp4mx_vendor_plan_destroy(void* plan) {
  destroy(static_cast<Plan*>(plan));
}

}  // extern "C"
