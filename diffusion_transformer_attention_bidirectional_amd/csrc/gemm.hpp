// Plain row-major GEMMs of the block path (the projections either side of attention),
// through hipBLASLt: bf16 / fp16 in and out, fp32 accumulation.  Host code.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

namespace krea {

// Workspace hipBLASLt may use per call (bytes).
constexpr size_t kGemmWorkspace = size_t(32) << 20;

// For b < batch:  Y_b = X_b W  (accumulate: Y_b += X_b W).
//   X_b: [M, K] row-major, row stride ldx, at X + b * sx (elements);
//   W:   [K, N] row-major (row stride N), shared by every b;
//   Y_b: [M, N] row-major, row stride ldy, at Y + b * sy.
// The first call of a shape picks the algorithm by timing hipBLASLt's candidates on the
// stream (and waits for them).  A plain product is timed in place, since its last run
// overwrites Y.  An accumulating one is timed without accumulation into `scratch`
// (batch x [M, N] contiguous) when given; without scratch it takes the heuristic's
// first choice.
// Returns false with `err` set when hipBLASLt refuses or fails.
bool gemm_rows(bool bf16, int64_t M, int64_t N, int64_t K, const void* X, int64_t ldx, int64_t sx, const void* W,
               void* Y, int64_t ldy, int64_t sy, int batch, bool accumulate, void* workspace, size_t workspace_bytes,
               hipStream_t stream, std::string* err, void* scratch = nullptr);

}  // namespace krea
