// M == 1 fused dequant-GEMV for the 4-bit block format (page "ONNX export,
// quantization and the browser runtime", section "Quantization", steps 1-2:
// y = x . w_hat + bias with w_hat = (q - z) * scale per 32-row block).
//
// The weights stream from HBM exactly once.  A lane owns 16 consecutive
// columns (8 bytes of a packed row) over the 32 rows of one K-block: 32
// independent 8-byte loads in flight per lane, 16 lanes reading 128
// contiguous bytes of each row.  Per packed word (8 weights) the inner loop
// issues 1 shift, 4 masks, 4 packed-fp16 subtractions and 8 v_fma_mix_f32
// (see common.h): each x * (q - z) product is exact and rounded once into
// fp32.  At the end of a block each column's sum is multiplied by its scale.
// Lane groups and waves that worked on other K-blocks of the same columns
// are summed through LDS; workgroups along K write partial sums to the
// workspace, which a second kernel adds in split order (splitk.h).
#include "common.h"
#include "launch.h"
#include "splitk.h"

namespace w4 {
namespace {

constexpr int kTN = kGemvTileCols;  // 256 columns per tile
constexpr int kLaneCols = 16;       // columns per lane


// The arguments the first loads depend on come first: the 14 dwords of x,
// Wq, scales, zeros, NB, N, tiles and bpw (the last two below 2^32: N / 256
// and at most 1024 blocks) arrive in SGPRs at wave launch (kernel-argument
// preloading), so no wave waits on an argument load.
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_fast(
    const float *__restrict__ x, const uint8_t *__restrict__ Wq, const float *__restrict__ scales,
    const uint8_t *__restrict__ zeros, int64_t NB, int64_t N, uint32_t tiles, uint32_t bpw,
    const float *__restrict__ bias, float *__restrict__ y, int64_t splits, int64_t npad,
    float *__restrict__ part) {
    constexpr int SLOTS = WAVES * kGemvGroups;
    __shared__ float red[SLOTS * kTN];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 4, li = lane & 15;
    const int slot = wave * kGemvGroups + grp;
    // the block index and the tile count fit 32 bits: a 32-bit division (a
    // 64-bit one is ~100 instructions ahead of the first load)
    const uint32_t bx = blockIdx.x, s32 = bx / tiles;
    const int64_t tile = bx - s32 * tiles, split = s32;
    const int64_t col = tile * kTN + li * kLaneCols;
    const int64_t half = N / 2;
    const int64_t b_end = min((split + 1) * bpw, NB);

    float yacc[kLaneCols];
#pragma unroll
    for (int j = 0; j < kLaneCols; ++j) yacc[j] = 0.0f;

    if (col < N) {
        for (int64_t b = split * bpw + slot; b < b_end; b += SLOTS) {
            const uint8_t *wp = Wq + b * kBlock * half + col / 2;
            u32x2_t wv[kBlock];
#pragma unroll
            for (int r = 0; r < kBlock; ++r) wv[r] = load_stream<u32x2_t>(wp + r * half);
            const f32x4_t *xp = reinterpret_cast<const f32x4_t *>(x + b * kBlock);
            f32x4_t xv[kBlock / 4];
#pragma unroll
            for (int i = 0; i < kBlock / 4; ++i) xv[i] = xp[i];
            const float *sp = scales + b * N + col;
            f32x4_t s4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) s4[i] = load_stream<f32x4_t>(sp + 4 * i);
            const u32x2_t zv = load_stream<u32x2_t>(zeros + b * half + col / 2);
            // keep every load above in flight before any arithmetic: the
            // scheduler would otherwise trade memory parallelism for registers
            __builtin_amdgcn_sched_barrier(0);
            const NibblePairs z0 = nibble_pairs(zv.x), z1 = nibble_pairs(zv.y);

            float acc[kLaneCols];
#pragma unroll
            for (int j = 0; j < kLaneCols; ++j) acc[j] = 0.0f;
#pragma unroll
            for (int r = 0; r < kBlock; ++r) {
                const float xr = xv[r >> 2][r & 3];
                fma_word(xr, wv[r].x, z0, acc);
                fma_word(xr, wv[r].y, z1, acc + 8);
            }
#pragma unroll
            for (int j = 0; j < kLaneCols; ++j)
                yacc[j] = __builtin_fmaf(s4[j >> 2][j & 3], acc[j], yacc[j]);
        }
    }

    // column c of the tile <-> lane li = c / 16, j = c % 16; stored [slot][j][li]
#pragma unroll
    for (int j = 0; j < kLaneCols; ++j) red[slot * kTN + j * 16 + li] = yacc[j] * nibble_unscale(j & 7);
    __syncthreads();

    for (int c = tid; c < kTN; c += 64 * WAVES) {
        const int ci = (c & 15) * 16 + (c >> 4);
        float v = 0.0f;
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) v += red[s * kTN + ci];
        const int64_t n = tile * kTN + c;
        if (splits == 1) {
            if (n < N) y[n] = bias ? v + bias[n] : v;
        } else {
            part[split * npad + n] = v;
        }
    }
}

// Any even N and any M: one thread per (row m, column pair j), sequential
// over K with w_hat formed exactly per weight.  Used where the fast kernels'
// alignment conditions do not hold (N % 16 != 0).
__global__ __launch_bounds__(256) void k_matmul_generic(const float *__restrict__ x, int64_t M,
                                                        int64_t K, const uint8_t *__restrict__ Wq,
                                                        const float *__restrict__ scales,
                                                        const uint8_t *__restrict__ zeros,
                                                        int64_t N, const float *__restrict__ bias,
                                                        float *__restrict__ y) {
    const int64_t half = N / 2;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= M * half) return;
    const int64_t m = i / half, j = i - m * half;
    const float *xm = x + m * K;
    float a0 = 0.0f, a1 = 0.0f;
    for (int64_t b = 0; b < K / kBlock; ++b) {
        const uint8_t zv = zeros[b * half + j];
        const float s0 = scales[b * N + 2 * j], s1 = scales[b * N + 2 * j + 1];
        const int z0 = zv & 15, z1 = zv >> 4;
        float c0 = 0.0f, c1 = 0.0f;
        for (int r = 0; r < kBlock; ++r) {
            const int64_t k = b * kBlock + r;
            const uint8_t qv = Wq[k * half + j];
            const float xv = xm[k];
            c0 = __builtin_fmaf(xv, (float)((int)(qv & 15) - z0), c0);
            c1 = __builtin_fmaf(xv, (float)((int)(qv >> 4) - z1), c1);
        }
        a0 = __builtin_fmaf(s0, c0, a0);
        a1 = __builtin_fmaf(s1, c1, a1);
    }
    if (bias) {
        a0 += bias[2 * j];
        a1 += bias[2 * j + 1];
    }
    y[m * N + 2 * j] = a0;
    y[m * N + 2 * j + 1] = a1;
}

__global__ __launch_bounds__(256) void k_bias_fill(const float *__restrict__ bias, int64_t M,
                                                   int64_t N, float *__restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= M * N) return;
    y[i] = bias ? bias[i % N] : 0.0f;
}

}  // namespace

hipError_t launch_bias_fill(const float *bias, int64_t M, int64_t N, float *y,
                            hipStream_t stream) {
    const int64_t total = M * N;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_bias_fill, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       bias, M, N, y);
    return hipGetLastError();
}

hipError_t launch_matmul_generic(const float *x, int64_t M, int64_t K, const uint8_t *Wq,
                                 const float *scales, const uint8_t *zeros, int64_t N,
                                 const float *bias, float *y, hipStream_t stream) {
    const int64_t total = M * (N / 2);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_matmul_generic, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, x, M, K, Wq, scales, zeros, N, bias, y);
    return hipGetLastError();
}

hipError_t launch_gemv(const GemvPlan &p, const float *x, int64_t K, const uint8_t *Wq,
                       const float *scales, const uint8_t *zeros, int64_t N, const float *bias,
                       float *y, void *workspace, hipStream_t stream) {
    switch (p.kind) {
    case GemvPlan::kEmpty:
        return hipSuccess;
    case GemvPlan::kBiasOnly:
        return launch_bias_fill(bias, 1, N, y, stream);
    case GemvPlan::kGeneric:
        return launch_matmul_generic(x, 1, K, Wq, scales, zeros, N, bias, y, stream);
    case GemvPlan::kFast:
        break;
    }
    float *part = static_cast<float *>(workspace);
    const dim3 grid((unsigned)(p.tiles * p.splits));
    const int64_t NB = K / kBlock;
#define W4_GEMV_CASE(WV)                                                                        \
    case WV:                                                                                    \
        hipLaunchKernelGGL(k_gemv_fast<WV>, grid, dim3(64 * WV), 0, stream, x, Wq, scales,       \
                           zeros, NB, N, (uint32_t)p.tiles, (uint32_t)p.blocks_per_wg, bias, y,  \
                           p.splits, p.npad,                                                    \
                           part);                                                               \
        break;
    switch (p.waves) {
        W4_GEMV_CASE(1)
        W4_GEMV_CASE(2)
        W4_GEMV_CASE(4)
    default:
        return hipErrorInvalidValue;
    }
#undef W4_GEMV_CASE
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_reduce(part, p.splits, 1, N, p.npad, bias, nullptr, 1.0f, y, stream);
}

}  // namespace w4
