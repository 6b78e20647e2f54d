// Second stage of the split-K kernels: a parallel, fixed-order sum of the
// partial planes (see splitk.h).
#include "launch.h"
#include "splitk.h"

#pragma clang fp contract(off)

namespace w4 {
namespace {

__global__ __launch_bounds__(256) void k_splitk_reduce(const float *__restrict__ part,
                                                       int64_t splits, int64_t rows, int64_t N,
                                                       int64_t npad,
                                                       const float *__restrict__ bias,
                                                       const float *__restrict__ col_scale,
                                                       float unit, float *__restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * N) return;
    const int64_t m = i / N, n = i - m * N;
    const float *p = part + m * npad + n;
    const int64_t plane = rows * npad;
    float v = 0.0f;
#pragma unroll 8
    for (int64_t s = 0; s < splits; ++s) v += p[s * plane];
    if (col_scale) v = (v * unit) * col_scale[n];
    if (bias) v += bias[n];
    y[i] = v;
}

}  // namespace

hipError_t launch_splitk_reduce(const float *part, int64_t splits, int64_t rows, int64_t N,
                                int64_t npad, const float *bias, const float *col_scale,
                                float unit, float *y, hipStream_t stream) {
    const int64_t total = rows * N;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       part, splits, rows, N, npad, bias, col_scale, unit, y);
    return hipGetLastError();
}

}  // namespace w4
