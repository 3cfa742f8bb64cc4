// Split-K dense GEMM (host side).  For shapes with too few output tiles to
// fill the GPU (few rows and few columns: decode-sized activations), the K
// chunks of each output tile (64x64 for at most 128 rows, else 128x96) are
// split over several workgroups.
// Each writes its FP32 partial of the tile (its chunks, promoted per chunk
// exactly as in the unsplit kernel) to a caller-provided workspace; a second
// kernel adds the partials in split order and writes D.  The promotion is
// linear in the chunk partials, so the split changes only the FP32 summation
// order.
#pragma once

#include "launch.h"

namespace fp8bs {

// k_gemm's layout mode for the split kernel (after GemmMode's values).
constexpr int kSplitK = 4;

// Splits for an M x N x K problem (1: no split) and the workspace bytes the
// split needs (0 without a split).
int32_t splitk_splits(int64_t M, int64_t N, int64_t K);
int64_t splitk_workspace_bytes(int64_t M, int64_t N, int64_t K);
// p.mode kDense.  Runs the split path when splitk_splits > 1 (ws must hold
// splitk_workspace_bytes), else the unsplit GEMM.
hipError_t launch_gemm_splitk(const GemmProblem& p, float* ws, hipStream_t stream);

}  // namespace fp8bs
