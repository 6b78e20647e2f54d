// Block quantizer/packer, unpacker and dequantizer for the 4-bit format of
// the page "ONNX export, quantization and the browser runtime", section
// "Quantization", step 2: blocks of 32 along K, one fp32 scale and one uint4
// zero point per block, w_hat = (q - z) * scale.  All three are bit-exact
// functions of their inputs.  H = true is the variant with the scale stored
// as binary16 (the same section's measurements table, "fp16 scales"): the
// fp32 scale (hi - lo) / 15 is rounded to binary16 (to nearest, ties to even)
// and the zero point and codes are taken against the stored value.
#include "common.h"
#include "launch.h"

// The quantizer's divisions and roundings must be the IEEE fp32 operations
// themselves: no contraction, correctly rounded division (the HIP default).
#pragma clang fp contract(off)

namespace w4 {
namespace {

__device__ __forceinline__ int clamp_code(float v, int lo, int hi) {
    if (v < (float)lo) return lo;
    if (v > (float)hi) return hi;
    return (int)v;
}

// Quantize one block column: 32 weights w[r] -> scale, zero point, codes.
// Returns false if a weight is not finite or the scale overflows.  With H the
// scale is stored as binary16 (h_out) and used at that value.
template <bool H>
__device__ __forceinline__ bool quantize_column(const float (&w)[kBlock], float &s_out,
                                                uint16_t &h_out, int &z_out,
                                                uint32_t (&q_out)[kBlock]) {
    float lo = 0.0f, hi = 0.0f;  // zero-inclusive range
    bool finite = true;
#pragma unroll
    for (int r = 0; r < kBlock; ++r) {
        const float v = w[r];
        finite &= __builtin_isfinite(v);
        if (v < lo) lo = v;
        if (v > hi) hi = v;
    }
    const float range = hi - lo;
    float s = range / 15.0f;
    finite &= __builtin_isfinite(s);
    if (H) {
        h_out = f32_to_f16_bits(s);
        finite &= (h_out & 0x7C00u) != 0x7C00u;  // binary16 overflow
        s = f16_bits_to_f32(h_out);
    }
    if (s == 0.0f || !finite) {
        s_out = finite ? 0.0f : s;
        z_out = 0;
#pragma unroll
        for (int r = 0; r < kBlock; ++r) q_out[r] = 0;
        return finite;
    }
    const int z = clamp_code(__builtin_rintf(-lo / s), 0, 15);
#pragma unroll
    for (int r = 0; r < kBlock; ++r) {
        const float t = __builtin_rintf(w[r] / s);
        q_out[r] = (uint32_t)clamp_code(t + (float)z, 0, 15);
    }
    s_out = s;
    z_out = z;
    return true;
}

// One thread per (K-block b, column pair j): reads 2 columns x 32 rows
// (8 bytes per row, adjacent threads adjacent), writes 32 packed bytes of Wq,
// two scales and one packed zero byte.
template <bool H>
__global__ __launch_bounds__(256) void k_quantize_pack(const float *__restrict__ W, int64_t K,
                                                       int64_t N, uint8_t *__restrict__ Wq,
                                                       void *__restrict__ scales,
                                                       uint8_t *__restrict__ zeros,
                                                       int *__restrict__ d_status) {
    const int64_t half = N / 2;
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t b = blockIdx.y;
    if (j >= half) return;
    float w0[kBlock], w1[kBlock];
    const float2 *src = reinterpret_cast<const float2 *>(W + b * kBlock * N) + j;
#pragma unroll
    for (int r = 0; r < kBlock; ++r) {
        const float2 v = src[r * half];
        w0[r] = v.x;
        w1[r] = v.y;
    }
    float s0, s1;
    uint16_t h0 = 0, h1 = 0;
    int z0, z1;
    uint32_t q0[kBlock], q1[kBlock];
    bool ok = quantize_column<H>(w0, s0, h0, z0, q0);
    ok &= quantize_column<H>(w1, s1, h1, z1, q1);
    if (!ok) set_status(d_status, W4_ERR_NONFINITE);
    uint8_t *dst = Wq + b * kBlock * half + j;
#pragma unroll
    for (int r = 0; r < kBlock; ++r) dst[r * half] = (uint8_t)(q0[r] | (q1[r] << 4));
    if (H)
        reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(scales) + b * N)[j] =
            (uint32_t)h0 | ((uint32_t)h1 << 16);
    else
        reinterpret_cast<float2 *>(static_cast<float *>(scales) + b * N)[j] = make_float2(s0, s1);
    zeros[b * half + j] = (uint8_t)(z0 | (z1 << 4));
}

// One thread per packed byte: q[2i], q[2i+1].  Covers Wq ([K, N/2] bytes) in
// the first `nq` threads and zeros ([K/32, N/2]) after them.
__global__ __launch_bounds__(256) void k_unpack(const uint8_t *__restrict__ Wq,
                                                const uint8_t *__restrict__ zeros, int64_t nq,
                                                int64_t nz, uint8_t *__restrict__ q,
                                                uint8_t *__restrict__ z) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nq) {
        const uint8_t v = Wq[i];
        reinterpret_cast<uchar2 *>(q)[i] = make_uchar2(v & 15, v >> 4);
    } else if (i < nq + nz) {
        const int64_t t = i - nq;
        const uint8_t v = zeros[t];
        reinterpret_cast<uchar2 *>(z)[t] = make_uchar2(v & 15, v >> 4);
    }
}

// One thread per packed byte (k, j): W_hat[k, 2j], W_hat[k, 2j+1].
template <bool H>
__global__ __launch_bounds__(256) void k_dequantize(const uint8_t *__restrict__ Wq,
                                                    const void *__restrict__ scales,
                                                    const uint8_t *__restrict__ zeros, int64_t K,
                                                    int64_t N, float *__restrict__ out) {
    const int64_t half = N / 2;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= K * half) return;
    const int64_t k = i / half, j = i - k * half;
    const int64_t b = k / kBlock;
    const uint8_t qv = Wq[i], zv = zeros[b * half + j];
    float2 s;
    if (H) {
        const uint32_t hh =
            reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(scales) + b * N)[j];
        s = make_float2(f16_bits_to_f32((uint16_t)hh), f16_bits_to_f32((uint16_t)(hh >> 16)));
    } else {
        s = reinterpret_cast<const float2 *>(static_cast<const float *>(scales) + b * N)[j];
    }
    // (q - z) is an exact small integer, so each output is one fp32 rounding
    const float d0 = (float)((int)(qv & 15) - (int)(zv & 15));
    const float d1 = (float)((int)(qv >> 4) - (int)(zv >> 4));
    reinterpret_cast<float2 *>(out)[i] = make_float2(d0 * s.x, d1 * s.y);
}

}  // namespace

hipError_t launch_quantize_pack(const float *W, int64_t K, int64_t N, uint8_t *Wq, void *scales,
                                bool f16, uint8_t *zeros, int *d_status, hipStream_t stream) {
    const int64_t half = N / 2, nb = K / kBlock;
    if (half == 0 || nb == 0) return hipSuccess;
    dim3 grid((unsigned)((half + 255) / 256), (unsigned)nb);
    if (f16)
        hipLaunchKernelGGL(k_quantize_pack<true>, grid, dim3(256), 0, stream, W, K, N, Wq, scales,
                           zeros, d_status);
    else
        hipLaunchKernelGGL(k_quantize_pack<false>, grid, dim3(256), 0, stream, W, K, N, Wq, scales,
                           zeros, d_status);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *Wq, const uint8_t *zeros, int64_t K, int64_t N,
                         uint8_t *q, uint8_t *z, hipStream_t stream) {
    const int64_t nq = K * (N / 2), nz = (K / kBlock) * (N / 2);
    const int64_t total = nq + nz;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_unpack, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, Wq,
                       zeros, nq, nz, q, z);
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t *Wq, const void *scales, bool f16,
                             const uint8_t *zeros, int64_t K, int64_t N, float *out,
                             hipStream_t stream) {
    const int64_t total = K * (N / 2);
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (f16)
        hipLaunchKernelGGL(k_dequantize<true>, grid, dim3(256), 0, stream, Wq, scales, zeros, K, N,
                           out);
    else
        hipLaunchKernelGGL(k_dequantize<false>, grid, dim3(256), 0, stream, Wq, scales, zeros, K,
                           N, out);
    return hipGetLastError();
}

}  // namespace w4
