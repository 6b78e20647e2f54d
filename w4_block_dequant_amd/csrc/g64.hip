// Group-64 affine variant of the 4-bit format (zero-tvm README, the kernel
// A/B table: "4-bit/group-64/affine").  Per group of 64 consecutive rows of a
// column: lo = min w, hi = max w, s = (hi - lo) / 15 and offset m = lo (both
// fp32), q = clamp(rint((w - lo) / s), 0, 15) (s = 0: q = 0), and
// w_hat = q * s + m with one rounding.  Codes are packed like the base
// format's; scales and minima are fp32 [K/64, N].  Bit-exact functions of
// their inputs.  The matmul runs in kmajor.hip (the GEMV's affine variant).
#include "common.h"
#include "launch.h"

// fp32 operations exactly as written: no contraction, correctly rounded
// division; the dequantization's single rounding is an explicit fma.
#pragma clang fp contract(off)

namespace w4 {
namespace {

constexpr int kGroup = 64;

__device__ __forceinline__ uint32_t g64_code(float w, float lo, float s) {
    if (s == 0.0f) return 0;
    const float t = __builtin_rintf((w - lo) / s);
    if (t < 0.0f) return 0;
    if (t > 15.0f) return 15;
    return (uint32_t)t;
}

// One thread per (group c, column pair j): the two columns' ranges in a first
// read of the 64 rows, their codes in a second (adjacent threads read
// adjacent 8-byte pairs, write adjacent bytes).
__global__ __launch_bounds__(256) void k_g64_quantize_pack(const float *__restrict__ W,
                                                           int64_t K, int64_t N,
                                                           uint8_t *__restrict__ Wq,
                                                           float *__restrict__ scales,
                                                           float *__restrict__ mins,
                                                           int *__restrict__ d_status) {
    const int64_t half = N / 2;
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t c = blockIdx.y;
    if (j >= half) return;
    const float2 *src = reinterpret_cast<const float2 *>(W + c * kGroup * N) + j;
    float2 v = src[0];
    float lo0 = v.x, hi0 = v.x, lo1 = v.y, hi1 = v.y;
    bool finite = true;
    for (int r = 0; r < kGroup; ++r) {
        v = src[r * half];
        finite &= __builtin_isfinite(v.x) && __builtin_isfinite(v.y);
        if (v.x < lo0) lo0 = v.x;
        if (v.x > hi0) hi0 = v.x;
        if (v.y < lo1) lo1 = v.y;
        if (v.y > hi1) hi1 = v.y;
    }
    const float s0 = (hi0 - lo0) / 15.0f, s1 = (hi1 - lo1) / 15.0f;
    finite &= __builtin_isfinite(s0) && __builtin_isfinite(s1);
    if (!finite) set_status(d_status, W4_ERR_NONFINITE);
    reinterpret_cast<float2 *>(scales + c * N)[j] = make_float2(s0, s1);
    reinterpret_cast<float2 *>(mins + c * N)[j] = make_float2(lo0, lo1);
    uint8_t *dst = Wq + c * kGroup * half + j;
    for (int r = 0; r < kGroup; ++r) {
        v = src[r * half];
        dst[r * half] = (uint8_t)(g64_code(v.x, lo0, s0) | (g64_code(v.y, lo1, s1) << 4));
    }
}

// One thread per packed byte (two weights of one row).
__global__ __launch_bounds__(256) void k_g64_dequantize(const uint8_t *__restrict__ Wq,
                                                        const float *__restrict__ scales,
                                                        const float *__restrict__ mins,
                                                        int64_t K, int64_t N,
                                                        float *__restrict__ W_hat) {
    const int64_t half = N / 2;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= K * half) return;
    const int64_t k = i / half, j = i - k * half;
    const uint8_t b = Wq[i];
    const int64_t gi = (k / kGroup) * N + 2 * j;
    const float2 s = *reinterpret_cast<const float2 *>(scales + gi);
    const float2 m = *reinterpret_cast<const float2 *>(mins + gi);
    reinterpret_cast<float2 *>(W_hat)[i] = make_float2(
        __builtin_fmaf((float)(b & 15), s.x, m.x), __builtin_fmaf((float)(b >> 4), s.y, m.y));
}

}  // namespace

hipError_t launch_g64_quantize_pack(const float *W, int64_t K, int64_t N, uint8_t *Wq,
                                    float *scales, float *mins, int *d_status,
                                    hipStream_t stream) {
    const int64_t half = N / 2, groups = K / kGroup;
    if (half == 0 || groups == 0) return hipSuccess;
    const dim3 grid((unsigned)((half + 255) / 256), (unsigned)groups);
    hipLaunchKernelGGL(k_g64_quantize_pack, grid, dim3(256), 0, stream, W, K, N, Wq, scales, mins,
                       d_status);
    return hipGetLastError();
}

hipError_t launch_g64_dequantize(const uint8_t *Wq, const float *scales, const float *mins,
                                 int64_t K, int64_t N, float *W_hat, hipStream_t stream) {
    const int64_t total = K * (N / 2);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_g64_dequantize, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, Wq, scales, mins, K, N, W_hat);
    return hipGetLastError();
}

}  // namespace w4
