// Deterministic split-K combination.
//
// A split-K kernel writes its fp32 partial sums to the workspace as
// part[s][m][n] (row stride npad, split stride rows * npad) with plain stores;
// a second kernel on the same stream then forms every output
// y[m, n] = sum_s part[s][m][n] (+ bias[n]) in split order, one thread per
// output.  No atomics, no counters and no ordering between workgroups of the
// first kernel; stream order makes the partials visible to the second.
#pragma once

#include "common.h"

namespace w4 {

// y[m, n] (row stride N) from `splits` partial planes of `rows` x npad floats;
// `scale` multiplies the sum before the bias is added (used by the int8 head
// to apply its fp16-subnormal unit and per-token scale: pass col_scale).
// `act` and `residual` are the fused epilogue (epilogue.h); with
// W4_ACT_SWIGLU, y has N / 2 columns.
hipError_t launch_splitk_reduce(const float *part, int64_t splits, int64_t rows, int64_t N,
                                int64_t npad, const float *bias, const float *col_scale,
                                float unit, float *y, hipStream_t stream,
                                const float *residual = nullptr, int act = W4_ACT_NONE);

}  // namespace w4
