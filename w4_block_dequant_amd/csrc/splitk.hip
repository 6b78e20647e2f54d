// Second stage of the split-K kernels: a parallel, fixed-order sum of the
// partial planes (see splitk.h).
#include "epilogue.h"
#include "launch.h"
#include "splitk.h"

#pragma clang fp contract(off)

namespace w4 {
namespace {

// Grid: x over groups of 4 columns (64 threads per workgroup, so that even a
// one-row reduce spreads over many compute units), y strides over rows (no
// index division).  Each thread adds 4 adjacent outputs with 16-byte reads of
// every plane (npad is a multiple of 4 and the planes are 256-byte aligned),
// in split order.
__global__ __launch_bounds__(64) void k_splitk_reduce(const float *__restrict__ part,
                                                       int splits, int64_t rows, int N,
                                                       int64_t npad,
                                                       const float *__restrict__ bias,
                                                       const float *__restrict__ col_scale,
                                                       float unit,
                                                       const float *residual, int act,
                                                       float *y) {
    const int n0 = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
    if (n0 >= N) return;
    const int64_t plane = rows * npad;
    for (int64_t m = blockIdx.y; m < rows; m += gridDim.y) {
        // bias and column scales of the 4 columns first (indices clamped to
        // N - 1, so the loads go out together, alongside the partial sums')
        float bj[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cj[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if (bias) {
#pragma unroll
            for (int j = 0; j < 4; ++j) bj[j] = bias[min(n0 + j, N - 1)];
        }
        if (col_scale) {
#pragma unroll
            for (int j = 0; j < 4; ++j) cj[j] = col_scale[min(n0 + j, N - 1)];
        }
        const float *p = part + m * npad + n0;
        // sixteen planes' loads in flight at a time (addresses clamped to the
        // last plane), then added in split order: the same sums as one plane
        // at a time, with one dependent round trip up to 16 splits
        f32x4_t v = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int s0 = 0; s0 < splits; s0 += 16) {
            f32x4_t r[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                r[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(
                    p + min(s0 + j, splits - 1) * plane));
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (s0 + j < splits) v += r[j];
        }
        float t[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float r = v[j];
            if (col_scale) r = (r * unit) * cj[j];
            if (bias) r += bj[j];
            t[j] = r;
        }
        if (act == W4_ACT_SWIGLU) {  // N even: pairs (n0, n0 + 1), (n0 + 2, n0 + 3)
            const int64_t no = N / 2;
#pragma unroll
            for (int j = 0; j < 4; j += 2)
                if (n0 + j < N) ep_store_glu(t[j], t[j + 1], residual, y, m * no + (n0 + j) / 2);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n0 + j < N) ep_store(t[j], act, residual, y, m * N + n0 + j);
        }
    }
}

}  // namespace

hipError_t launch_splitk_reduce(const float *part, int64_t splits, int64_t rows, int64_t N,
                                int64_t npad, const float *bias, const float *col_scale,
                                float unit, float *y, hipStream_t stream, const float *residual,
                                int act) {
    if (rows == 0 || N == 0) return hipSuccess;
    const int64_t groups = (N + 3) / 4;
    const dim3 grid((unsigned)((groups + 63) / 64), (unsigned)(rows < 65535 ? rows : 65535));
    hipLaunchKernelGGL(k_splitk_reduce, grid, dim3(64), 0, stream, part, (int)splits, rows,
                       (int)N, npad, bias, col_scale, unit, residual, act, y);
    return hipGetLastError();
}

}  // namespace w4
