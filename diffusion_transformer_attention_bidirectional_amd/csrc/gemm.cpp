// hipBLASLt calls of the block path.  hipBLASLt is column-major: a row-major Y = X W is
// the column-major Y^T = W^T X^T, where a row-major [R, C] array with row stride ld is
// the column-major [C, R] array with leading dimension ld -- so no operand is
// transposed: A = W ([N, K], ld N), B = X ([K, M], ld ldx), C = D = Y ([N, M], ld ldy).
#include "gemm.hpp"

#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

namespace krea {
namespace {

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;  // one per device, for the process' lifetime

// device, dtype, shape, strides, batch, accumulate, workspace bytes: an algorithm chosen
// under a larger workspace may need more than a later call provides
using AlgoKey =
    std::tuple<int, bool, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int, bool, size_t>;
std::map<AlgoKey, hipblasLtMatmulAlgo_t> g_algos;  // the heuristic's first choice per call shape

bool check(hipblasStatus_t s, const char* what, std::string* err) {
  if (s == HIPBLAS_STATUS_SUCCESS) return true;
  if (err) *err = std::string("hipBLASLt ") + what + " failed (status " + std::to_string((int)s) + ")";
  return false;
}

// Descriptors of one call, released on scope exit.
struct Descs {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  ~Descs() {
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (c) hipblasLtMatrixLayoutDestroy(c);
    if (b) hipblasLtMatrixLayoutDestroy(b);
    if (a) hipblasLtMatrixLayoutDestroy(a);
    if (op) hipblasLtMatmulDescDestroy(op);
  }
};

bool batched(hipblasLtMatrixLayout_t l, int batch, int64_t stride, std::string* err) {
  if (batch <= 1) return true;
  const int32_t n = batch;
  return check(hipblasLtMatrixLayoutSetAttribute(l, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &n, sizeof(n)),
               "layout batch count", err) &&
         check(hipblasLtMatrixLayoutSetAttribute(l, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &stride,
                                                 sizeof(stride)),
               "layout batch stride", err);
}

// Candidates timed on the first call of a shape, and launches per candidate timing.
constexpr int kCandidates = 12;
constexpr int kTimedRuns = 3;

// The fastest of hipBLASLt's candidates for the described product, run with beta = 0 on
// `out` (laid out as `c`).  Candidates that fail to launch are skipped.
bool fastest(hipblasLtHandle_t h, const Descs& d, hipblasLtMatrixLayout_t c, const void* W, const void* X,
             void* out, void* workspace, size_t workspace_bytes, hipStream_t stream,
             const hipblasLtMatmulHeuristicResult_t* res, int found, hipblasLtMatmulAlgo_t* best,
             std::string* err) {
  *best = res[0].algo;
  if (found < 2) return true;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) hipEventDestroy(e0);
    if (err) *err = "hipEventCreate failed";
    return false;
  }
  const float alpha = 1.0f, beta = 0.0f;
  float best_ms = 0.f;
  bool have = false, ok = true;
  for (int i = 0; i < found && ok; ++i) {
    if (res[i].state != HIPBLAS_STATUS_SUCCESS || res[i].workspaceSize > workspace_bytes) continue;
    auto run = [&]() {
      return hipblasLtMatmul(h, d.op, &alpha, W, d.a, X, d.b, &beta, out, c, out, c, &res[i].algo, workspace,
                             workspace_bytes, stream) == HIPBLAS_STATUS_SUCCESS;
    };
    if (!run()) continue;  // this candidate does not take these operands
    bool timed = hipEventRecord(e0, stream) == hipSuccess;
    for (int r = 0; r < kTimedRuns && timed; ++r) timed = run();
    timed = timed && hipEventRecord(e1, stream) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
    float ms = 0.f;
    if (!timed || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
      ok = false;
      break;
    }
    if (!have || ms < best_ms) {
      best_ms = ms;
      *best = res[i].algo;
      have = true;
    }
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  if (!ok && err) *err = "timing the hipBLASLt candidates failed";
  return ok;
}

}  // namespace

bool gemm_rows(bool bf16, int64_t M, int64_t N, int64_t K, const void* X, int64_t ldx, int64_t sx, const void* W,
               void* Y, int64_t ldy, int64_t sy, int batch, bool accumulate, void* workspace, size_t workspace_bytes,
               hipStream_t stream, std::string* err, void* scratch) {
  if (M <= 0 || N <= 0 || K <= 0 || batch <= 0) return true;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    if (err) *err = "hipGetDevice failed";
    return false;
  }
  hipblasLtHandle_t h = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_handles.find(dev);
    if (it == g_handles.end()) {
      if (!check(hipblasLtCreate(&h), "create", err)) return false;
      g_handles[dev] = h;
    } else {
      h = it->second;
    }
  }
  const hipDataType dt = bf16 ? HIP_R_16BF : HIP_R_16F;
  Descs d;
  const int32_t op_n = HIPBLAS_OP_N;
  if (!check(hipblasLtMatmulDescCreate(&d.op, HIPBLAS_COMPUTE_32F, HIP_R_32F), "matmul desc", err) ||
      !check(hipblasLtMatmulDescSetAttribute(d.op, HIPBLASLT_MATMUL_DESC_TRANSA, &op_n, sizeof(op_n)), "trans A",
             err) ||
      !check(hipblasLtMatmulDescSetAttribute(d.op, HIPBLASLT_MATMUL_DESC_TRANSB, &op_n, sizeof(op_n)), "trans B",
             err) ||
      !check(hipblasLtMatrixLayoutCreate(&d.a, dt, N, K, N), "layout W", err) ||
      !check(hipblasLtMatrixLayoutCreate(&d.b, dt, K, M, ldx), "layout X", err) ||
      !check(hipblasLtMatrixLayoutCreate(&d.c, dt, N, M, ldy), "layout Y", err) || !batched(d.a, batch, 0, err) ||
      !batched(d.b, batch, sx, err) || !batched(d.c, batch, sy, err))
    return false;
  const AlgoKey key{dev, bf16, M, N, K, ldx, sx, ldy, sy, batch, accumulate, workspace_bytes};
  hipblasLtMatmulAlgo_t algo;
  bool have = false;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_algos.find(key);
    if (it != g_algos.end()) {
      algo = it->second;
      have = true;
    }
  }
  if (!have) {
    const uint64_t wsb = workspace_bytes;
    if (!check(hipblasLtMatmulPreferenceCreate(&d.pref), "preference", err) ||
        !check(hipblasLtMatmulPreferenceSetAttribute(d.pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb,
                                                     sizeof(wsb)),
               "preference workspace", err))
      return false;
    hipblasLtMatmulHeuristicResult_t res[kCandidates];
    int found = 0;
    if (!check(hipblasLtMatmulAlgoGetHeuristic(h, d.op, d.a, d.b, d.c, d.c, d.pref, kCandidates, res, &found),
               "heuristic", err))
      return false;
    if (found < 1) {
      if (err) *err = "hipBLASLt has no algorithm for this GEMM";
      return false;
    }
    if (!accumulate) {
      if (!fastest(h, d, d.c, W, X, Y, workspace, workspace_bytes, stream, res, found, &algo, err)) return false;
    } else if (scratch != nullptr) {
      // the same product without accumulation, into a contiguous scratch of Y's shape
      hipblasLtMatrixLayout_t ct = nullptr;
      bool ok = check(hipblasLtMatrixLayoutCreate(&ct, dt, N, M, N), "layout scratch", err) &&
                batched(ct, batch, N * M, err) &&
                fastest(h, d, ct, W, X, scratch, workspace, workspace_bytes, stream, res, found, &algo, err);
      if (ct) hipblasLtMatrixLayoutDestroy(ct);
      if (!ok) return false;
    } else {
      algo = res[0].algo;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    g_algos[key] = algo;
  }
  const float alpha = 1.0f, beta = accumulate ? 1.0f : 0.0f;
  return check(hipblasLtMatmul(h, d.op, &alpha, W, d.a, X, d.b, &beta, Y, d.c, Y, d.c, &algo, workspace,
                               workspace_bytes, stream),
               "matmul", err);
}

}  // namespace krea
