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
// Returns false with `err` set when hipBLASLt refuses or fails.
bool gemm_rows(bool bf16, int64_t M, int64_t N, int64_t K, const void* X, int64_t ldx, int64_t sx, const void* W,
               void* Y, int64_t ldy, int64_t sy, int batch, bool accumulate, void* workspace, size_t workspace_bytes,
               hipStream_t stream, std::string* err);

}  // namespace krea
