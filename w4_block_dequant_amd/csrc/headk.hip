// int8 tied LM head on a K-major copy of the table (page "ONNX export,
// quantization and the browser runtime", section "Quantization", steps 3-4:
// one int8 table with one fp32 scale per token, read directly by the head for
// the last position and gathered for the token lookup).
//
// Layout: Qt int8 [N, ldt], Qt[n, k] = Q[k, n], rows padded with zeros to
// ldt >= K (ldt % 16 == 0).  Row n is token n's embedding, contiguous, which
// is what both the lookup and the head want: the head reads every row once
// from start to end.
//
// Head arithmetic: fp32 on the vector ALUs, exact in its operands.  Each
// signed code becomes an fp32 number in one instruction (a byte-select
// conversion), and the logit is hs[n] * sum_k x[k] Q[k, n] with every product
// formed by an fp32 FMA: no quantization of x, so the result is within the
// matmul bound for any finite input.  A row of x with a non-finite entry gives
// NaN logits for that row.
#include "common.h"
#include "launch.h"

namespace w4 {
namespace {

// Relayout Q [K, ldq] -> Qt [N, ldt] through a 64 x 64 byte tile in LDS;
// columns ldt > k >= K of Qt are written as zeros.
__global__ __launch_bounds__(256) void k_head_prepack(const int8_t *__restrict__ Q, int64_t K,
                                                      int64_t N, int64_t ldq,
                                                      int8_t *__restrict__ Qt, int64_t ldt) {
    __shared__ int8_t tile[64][65];
    const int64_t k0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4
    for (int r = ty; r < 64; r += 4) {
        const int64_t k = k0 + r, n = n0 + tx;
        tile[r][tx] = (k < K && n < N) ? Q[k * ldq + n] : (int8_t)0;
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {
        const int64_t n = n0 + r, k = k0 + tx;
        if (n < N && k < ldt) Qt[n * ldt + k] = tile[tx][r];
    }
}

// Token lookup from Qt: out[t, k] = fl32(Qt[tok, k] * hs[tok]), one thread
// per output; a row is contiguous.
__global__ __launch_bounds__(256) void k_embed_kmajor(const int64_t *__restrict__ tokens,
                                                      int64_t T, const int8_t *__restrict__ Qt,
                                                      int64_t ldt, const float *__restrict__ hs,
                                                      int64_t K, int64_t N,
                                                      float *__restrict__ out,
                                                      int *__restrict__ d_status) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T * K) return;
    const int64_t t = i / K, k = i - t * K;
    const int64_t tok = tokens[t];
    if (tok < 0 || tok >= N) {
        if (k == 0) set_status(d_status, W4_ERR_BAD_SHAPE);
        out[i] = 0.0f;
        return;
    }
    out[i] = (float)Qt[tok * ldt + k] * hs[tok];
}

// One wave takes 4 RPW tokens: in round r, lane group g = lane / 16 owns
// token t0 + 4 r + g, and lane c = lane % 16 owns bytes 16 c + 256 i of each
// 256 CH-wide slice of the token's row (i < CH): one 16-byte load per chunk,
// so a load instruction reads four 256-byte runs of four rows.  The rows of x
// pass through LDS in groups of RB; every lane reads its 16 activations per
// chunk from there.  Each chunk's 16 products are summed on their own and
// then added to the lane's total (short fp32 chains), and the 16 lanes of a
// token add their totals in a fixed butterfly: deterministic results.  Past
// K a lane re-reads a valid chunk whose activations are zero; past N it
// re-reads the last token and stores nothing.
template <int CH, int RPW>
__global__ __launch_bounds__(256) void k_head_fp32(const float *__restrict__ x, int M, int K,
                                                   const int8_t *__restrict__ Qt, int ldt,
                                                   const float *__restrict__ hs, int N, int RB,
                                                   float *__restrict__ logits) {
    extern __shared__ f32x4_t xs[];  // [RB][K / 4]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int t0 = (blockIdx.x * 4 + wave) * (4 * RPW);
    constexpr int SW = 256 * CH;  // slice width in k
    const int nsl = (K + SW - 1) / SW;
    const int K4 = K / 4;

    uint32_t roff[RPW];
    float hsv[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int tc = min(t0 + 4 * r + g, N - 1);
        roff[r] = (uint32_t)tc * (uint32_t)ldt;
    }
    u32x4_t w[RPW][CH];
    auto load_w = [&](int sl) {
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int k = min(sl * SW + 256 * i + 16 * c, K - 16);
                w[r][i] = load_stream<u32x4_t>(Qt + (roff[r] + (uint32_t)k));
            }
    };
    if (nsl == 1) load_w(0);  // the whole row of every token in flight before anything else
#pragma unroll
    for (int r = 0; r < RPW; ++r) hsv[r] = hs[min(t0 + 4 * r + g, N - 1)];

    for (int m0 = 0; m0 < M; m0 += RB) {
        const int rows = min(RB, M - m0);
        __syncthreads();  // the previous group's reads are done
        const f32x4_t *xr = reinterpret_cast<const f32x4_t *>(x + (size_t)m0 * K);
        for (int i = tid; i < rows * K4; i += 256) xs[i] = xr[i];
        __syncthreads();
        for (int rr = 0; rr < rows; ++rr) {
            float acc[RPW];
#pragma unroll
            for (int r = 0; r < RPW; ++r) acc[r] = 0.0f;
            bool fin = true;
            for (int sl = 0; sl < nsl; ++sl) {
                if (nsl > 1) load_w(sl);
                float xv[CH][16];
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const int k = sl * SW + 256 * i + 16 * c;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4_t v = k < K ? xs[rr * K4 + k / 4 + q] : f32x4_t{0.f, 0.f, 0.f, 0.f};
                        xv[i][4 * q + 0] = v.x;
                        xv[i][4 * q + 1] = v.y;
                        xv[i][4 * q + 2] = v.z;
                        xv[i][4 * q + 3] = v.w;
                    }
#pragma unroll
                    for (int j = 0; j < 16; ++j) fin &= __builtin_isfinite(xv[i][j]);
                }
#pragma unroll
                for (int r = 0; r < RPW; ++r)
#pragma unroll
                    for (int i = 0; i < CH; ++i) {
                        const uint32_t ws[4] = {w[r][i].x, w[r][i].y, w[r][i].z, w[r][i].w};
                        float t = 0.0f;
#pragma unroll
                        for (int d = 0; d < 4; ++d)
#pragma unroll
                            for (int b = 0; b < 4; ++b)
                                t = __builtin_fmaf(xv[i][4 * d + b],
                                                   (float)(int)(int8_t)(ws[d] >> (8 * b)), t);
                        acc[r] += t;
                    }
            }
            const bool row_ok = __all(fin);
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                float v = acc[r];
                v += __shfl_xor(v, 8);
                v += __shfl_xor(v, 4);
                v += __shfl_xor(v, 2);
                v += __shfl_xor(v, 1);
                const int t = t0 + 4 * r + g;
                if (c == 0 && t < N)
                    logits[(size_t)(m0 + rr) * N + t] = row_ok ? v * hsv[r] : __builtin_nanf("");
            }
        }
    }
}

}  // namespace

hipError_t launch_head_prepack(const int8_t *Q, int64_t K, int64_t N, int64_t ldq, int8_t *Qt,
                               int64_t ldt, hipStream_t stream) {
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((ldt + 63) / 64));
    hipLaunchKernelGGL(k_head_prepack, grid, dim3(256), 0, stream, Q, K, N, ldq, Qt, ldt);
    return hipGetLastError();
}

hipError_t launch_embed_kmajor(const int64_t *tokens, int64_t T, const int8_t *Qt, int64_t ldt,
                               const float *hs, int64_t K, int64_t N, float *out, int *d_status,
                               hipStream_t stream) {
    const int64_t total = T * K;
    hipLaunchKernelGGL(k_embed_kmajor, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       tokens, T, Qt, ldt, hs, K, N, out, d_status);
    return hipGetLastError();
}

// Rows of x staged per workgroup: at most 48 KB of LDS, at most 16 rows.
static int head_rows_per_group(int64_t M, int64_t K) {
    int64_t rb = 12288 / K;
    if (rb > 16) rb = 16;
    if (rb < 1) rb = 1;
    if (rb > M) rb = M;
    return (int)rb;
}

static hipError_t launch_head_fp32(const float *x, int64_t M, int64_t K, const int8_t *Qt,
                                   int64_t ldt, const float *hs, int64_t N, float *logits,
                                   hipStream_t stream) {
    const int rb = head_rows_per_group(M, K);
    const size_t shm = (size_t)rb * K * sizeof(float);
    constexpr int RPW = 4;  // 4 RPW = 16 tokens per wave, 64 per workgroup
    const dim3 grid((unsigned)((N + 16 * RPW - 1) / (16 * RPW)));
#define W4_HF(CHV)                                                                                \
    hipLaunchKernelGGL((k_head_fp32<CHV, RPW>), grid, dim3(256), shm, stream, x, (int)M, (int)K,  \
                       Qt, (int)ldt, hs, (int)N, rb, logits)
    if (K <= 256) W4_HF(1);
    else if (K <= 512) W4_HF(2);
    else if (K <= 768) W4_HF(3);
    else W4_HF(4);
#undef W4_HF
    return hipGetLastError();
}

hipError_t launch_head_logits_kmajor(const float *x, int64_t K, const int8_t *Qt, int64_t ldt,
                                     const float *hs, int64_t N, float *logits,
                                     hipStream_t stream) {
    return launch_head_fp32(x, 1, K, Qt, ldt, hs, N, logits, stream);
}

size_t head_rows_workspace(int64_t M, int64_t K) {
    (void)M;
    (void)K;
    return 0;
}

hipError_t launch_head_rows_kmajor(const float *x, int64_t M, int64_t K, const int8_t *Qt,
                                   int64_t ldt, const float *hs, int64_t N, float *logits,
                                   void *workspace, hipStream_t stream) {
    (void)workspace;
    return launch_head_fp32(x, M, K, Qt, ldt, hs, N, logits, stream);
}

}  // namespace w4
