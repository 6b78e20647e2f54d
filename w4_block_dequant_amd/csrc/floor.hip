// Streaming-read reference (include/w4.h, w4_read_bytes): the launch floor
// the benchmark sets beside the decode GEMV.  Each lane reads L 16-byte
// pieces with streaming (non-temporal) loads, as the GEMV reads its codes,
// and each wave writes the XOR of everything it read (a register-only lane
// reduction, no LDS, no barrier), so no load is dead.  Nothing else: no
// activations, no dequantization arithmetic.
#include "common.h"

namespace w4 {
namespace {

// XOR over the 64 lanes of a wave in DPP steps; the result is valid in lane 63
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_xor(uint32_t v) {
    return v ^ (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

template <int L>
__global__ __launch_bounds__(256) void k_read_bytes(const u32x4_t *__restrict__ src, int64_t n16,
                                                    uint32_t *__restrict__ out) {
    const int64_t lanes = (int64_t)gridDim.x * 256;
    const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    u32x4_t v[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const int64_t i = i0 + lanes * j;
        v[j] = load_stream<u32x4_t>(src + (i < n16 ? i : n16 - 1));
    }
    uint32_t a = 0;
#pragma unroll
    for (int j = 0; j < L; ++j)
        if (i0 + lanes * j < n16) a ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    a = dpp_xor<0xB1, 0xF>(a);   // quad_perm [1,0,3,2]
    a = dpp_xor<0x4E, 0xF>(a);   // quad_perm [2,3,0,1]
    a = dpp_xor<0x124, 0xF>(a);  // row_ror:4
    a = dpp_xor<0x128, 0xF>(a);  // row_ror:8
    a = dpp_xor<0x142, 0xA>(a);  // row_bcast:15
    a = dpp_xor<0x143, 0xC>(a);  // row_bcast:31
    if ((threadIdx.x & 63) == 63) out[(int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = a;
}

}  // namespace

int64_t read_bytes_groups(int64_t bytes, int loads) {
    const int64_t per = (int64_t)256 * 16 * loads;
    return (bytes + per - 1) / per;
}

int64_t read_bytes_words(int64_t bytes, int loads) { return 4 * read_bytes_groups(bytes, loads); }

hipError_t launch_read_bytes(const void *src, int64_t bytes, int loads, uint32_t *out,
                             hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const dim3 grid((unsigned)read_bytes_groups(bytes, loads));
    const u32x4_t *s = static_cast<const u32x4_t *>(src);
    switch (loads) {
    case 4: hipLaunchKernelGGL((k_read_bytes<4>), grid, dim3(256), 0, stream, s, n16, out); break;
    case 6: hipLaunchKernelGGL((k_read_bytes<6>), grid, dim3(256), 0, stream, s, n16, out); break;
    case 8: hipLaunchKernelGGL((k_read_bytes<8>), grid, dim3(256), 0, stream, s, n16, out); break;
    case 12: hipLaunchKernelGGL((k_read_bytes<12>), grid, dim3(256), 0, stream, s, n16, out); break;
    case 16: hipLaunchKernelGGL((k_read_bytes<16>), grid, dim3(256), 0, stream, s, n16, out); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace w4
