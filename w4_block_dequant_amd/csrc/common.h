// Device helpers shared by the gfx950 kernels of the 4-bit block-dequant
// matmul and the int8 head.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4.h"

namespace w4 {

constexpr int kBlock = 32;  // rows per quantization block along K

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Streaming load (read once: marked non-temporal so it does not displace
// reused lines in the caches).
template <class T>
__device__ __forceinline__ T load_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const T *>(p));
}

__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// Nibble pairs as fp16 subnormals.
//
// A 32-bit word of packed codes holds 8 consecutive columns, nibble i in bits
// 4i..4i+3.  Masking a word with 0x000F000F leaves nibbles 0 and 4 in the low
// bits of the two 16-bit halves: read as fp16 they are the subnormals
// q * 2^-24.  Masking with 0x00F000F0 leaves nibbles 1 and 5 four bits higher:
// q * 2^-20.  The word shifted right by 8 gives nibbles 2/6 and 3/7 the same
// way.  Subtracting the zero point's pair, masked identically, is exact in
// fp16 ((q - z) * 2^-24 is a multiple of the smallest subnormal and below the
// normal range), and v_fma_mix_f32 widens the selected half exactly.  So each
// product x * (q - z) is formed exactly and rounded once into the fp32
// accumulator, two weights per packed-fp16 subtraction.  The power of two is
// undone per column at the end (2^24 for even nibble positions, 2^20 for odd).
// fp16 and fp32 subnormals are enabled for HIP kernels on gfx950 (denorm mode 3).
struct NibblePairs {
    half2_t p[4];  // columns (0,4), (1,5), (2,6), (3,7) of the word
};

__device__ __forceinline__ NibblePairs nibble_pairs(uint32_t v) {
    const uint32_t hi = v >> 8;
    NibblePairs r;
    r.p[0] = as_half2(v & 0x000F000Fu);
    r.p[1] = as_half2(v & 0x00F000F0u);
    r.p[2] = as_half2(hi & 0x000F000Fu);
    r.p[3] = as_half2(hi & 0x00F000F0u);
    return r;
}

// acc[c] += x * (q[c] - z[c]) for the 8 columns of one packed word; acc is
// indexed by column within the word, in the scaled units described above.
__device__ __forceinline__ void fma_word(float x, uint32_t qword, const NibblePairs &z,
                                         float *acc) {
    const NibblePairs q = nibble_pairs(qword);
    half2_t d[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) d[m] = q.p[m] - z.p[m];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        acc[m] = __builtin_fmaf(x, (float)d[m].x, acc[m]);
        acc[m + 4] = __builtin_fmaf(x, (float)d[m].y, acc[m + 4]);
    }
}

// binary16 scales: fp32 -> binary16 bits (round to nearest even; v_cvt_f16_f32
// keeps subnormals, overflows to infinity) and back (exact).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// Undo the fp16-subnormal scaling of column c (0..7) of a packed word.
__device__ __forceinline__ constexpr float nibble_unscale(int c) {
    return (c & 1) ? 1048576.0f /* 2^20 */ : 16777216.0f /* 2^24 */;
}

__device__ __forceinline__ void set_status(int *d_status, int code) {
    if (d_status) atomicCAS(d_status, 0, code);
}

}  // namespace w4
