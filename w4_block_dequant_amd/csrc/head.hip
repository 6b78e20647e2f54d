// int8 tied LM head (page "ONNX export, quantization and the browser
// runtime", section "Quantization", steps 3-4): one int8 table [K, ldq] with
// one fp32 scale per token column, read directly by the head for the last
// position only, and gathered by column for the token lookup.
#include "common.h"
#include "launch.h"
#include "splitk.h"

#pragma clang fp contract(off)

namespace w4 {
namespace {

constexpr int kTN = 256;       // columns per tile
constexpr int kLaneCols = 16;  // columns (bytes) per lane
constexpr int kRows = 32;      // rows per lane group per pass

__device__ __forceinline__ int clamp_code(float v, int lo, int hi) {
    if (v < (float)lo) return lo;
    if (v > (float)hi) return hi;
    return (int)v;
}

// Per-token quantizer: one thread per column n (adjacent threads adjacent
// columns, so every row access is coalesced).  hs = max|E| / 127 with a
// correctly rounded fp32 division; Q = clamp(rint(E / hs), -127, 127).
__global__ __launch_bounds__(256) void k_head_quantize(const float *__restrict__ E, int64_t K,
                                                       int64_t N, int64_t ldq,
                                                       int8_t *__restrict__ Q,
                                                       float *__restrict__ hs,
                                                       int *__restrict__ d_status) {
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= ldq) return;
    if (n >= N) {  // padding column
        for (int64_t k = 0; k < K; ++k) Q[k * ldq + n] = 0;
        return;
    }
    float amax = 0.0f;
    bool finite = true;
    for (int64_t k = 0; k < K; ++k) {
        const float v = E[k * N + n];
        finite &= __builtin_isfinite(v);
        const float a = __builtin_fabsf(v);
        if (a > amax) amax = a;
    }
    const float s = amax / 127.0f;
    if (!finite || !__builtin_isfinite(s)) set_status(d_status, W4_ERR_NONFINITE);
    hs[n] = s;
    for (int64_t k = 0; k < K; ++k) {
        int qv = 0;
        if (s != 0.0f) qv = clamp_code(__builtin_rintf(E[k * N + n] / s), -127, 127);
        Q[k * ldq + n] = (int8_t)qv;
    }
}

// Token lookup: out[t, k] = fl32(Q[k, tok] * hs[tok]); one thread per output.
__global__ __launch_bounds__(256) void k_embed(const int64_t *__restrict__ tokens, int64_t T,
                                               const int8_t *__restrict__ Q, int64_t ldq,
                                               const float *__restrict__ hs, int64_t K, int64_t N,
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
    out[i] = (float)Q[k * ldq + tok] * hs[tok];
}

struct __attribute__((aligned(4))) Dword4 {
    uint32_t v[4];
};

// 16 table bytes of one row for one lane, from a byte offset `a` into Q.
// ALIGNED: ldq % 16 == 0, so `a` is 16-byte aligned and the load is in bounds.
// Otherwise a 20-byte window of dword-aligned loads is shifted into place;
// near the end of the table, where the window would pass the last byte, the
// bytes are read one by one.
template <bool ALIGNED>
__device__ __forceinline__ u32x4_t load_row16(const int8_t *__restrict__ Q, int64_t a,
                                              int64_t total) {
    if (ALIGNED) return load_stream<u32x4_t>(Q + a);
    const int sh = (int)(a & 3);
    const int64_t a0 = a - sh;
    uint32_t d[5];
    if (a0 + 20 <= total) {
        const Dword4 w = *reinterpret_cast<const Dword4 *>(Q + a0);
        d[0] = w.v[0];
        d[1] = w.v[1];
        d[2] = w.v[2];
        d[3] = w.v[3];
        d[4] = *reinterpret_cast<const uint32_t *>(Q + a0 + 16);
    } else {
        const uint8_t *p = reinterpret_cast<const uint8_t *>(Q);
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            uint32_t v = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int64_t o = a0 + 4 * i + b;
                if (o < total) v |= (uint32_t)p[o] << (8 * b);
            }
            d[i] = v;
        }
    }
    u32x4_t r;
    r.x = __builtin_amdgcn_alignbyte(d[1], d[0], sh);
    r.y = __builtin_amdgcn_alignbyte(d[2], d[1], sh);
    r.z = __builtin_amdgcn_alignbyte(d[3], d[2], sh);
    r.w = __builtin_amdgcn_alignbyte(d[4], d[3], sh);
    return r;
}

// acc[c] += x * q[c] * 2^-24 for the 4 signed bytes of a word.  XOR 0x80
// makes each byte u = q + 128 in [1, 255]; two bytes masked into the halves
// are the fp16 subnormals u * 2^-24, and subtracting 128 * 2^-24 is exact,
// leaving q * 2^-24.  Byte c of the word is column c.
__device__ __forceinline__ void fma_i8_word(float x, uint32_t w, float *acc) {
    const uint32_t u = w ^ 0x80808080u;
    const half2_t bias = as_half2(0x00800080u);
    const half2_t p02 = as_half2(u & 0x00FF00FFu) - bias;
    const half2_t p13 = as_half2((u >> 8) & 0x00FF00FFu) - bias;
    acc[0] = __builtin_fmaf(x, (float)p02.x, acc[0]);
    acc[2] = __builtin_fmaf(x, (float)p02.y, acc[2]);
    acc[1] = __builtin_fmaf(x, (float)p13.x, acc[1]);
    acc[3] = __builtin_fmaf(x, (float)p13.y, acc[3]);
}

// logits[n] = hs[n] * sum_k x[k] * Q[k, n].  The per-token scale factors out
// of the sum: fl32(Q * hs) differs from Q * hs by at most 2^-24 relative.
// A lane owns 16 columns and the 32 rows of one row block; 16 lanes cover a
// 256-column tile, the 4 lane groups of a wave take 4 row blocks.  x for the
// workgroup's rows is staged once in LDS.
template <int WAVES, bool ALIGNED>
__global__ __launch_bounds__(64 * WAVES) void k_head_logits(
    const float *__restrict__ x, int64_t K, const int8_t *__restrict__ Q, int64_t ldq,
    const float *__restrict__ hs, int64_t N, float *__restrict__ logits, int64_t tiles,
    int64_t splits, int64_t rows_per_wg, int64_t npad, float *__restrict__ part) {
    constexpr int SLOTS = WAVES * kGemvGroups;
    extern __shared__ float smem[];
    float *red = smem;                    // [SLOTS * kTN]
    float *xs = smem + SLOTS * kTN;       // [rows_per_wg]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int grp = lane >> 4, li = lane & 15;
    const int slot = wave * kGemvGroups + grp;
    const int64_t tile = blockIdx.x % tiles, split = blockIdx.x / tiles;
    const int64_t col = tile * kTN + li * kLaneCols;
    const int64_t r_begin = split * rows_per_wg;
    const int64_t r_end = min(r_begin + rows_per_wg, K);
    const int64_t total = K * ldq;

    for (int64_t r = r_begin + tid; r < r_end; r += 64 * WAVES) xs[r - r_begin] = x[r];
    __syncthreads();

    float acc[kLaneCols];
#pragma unroll
    for (int j = 0; j < kLaneCols; ++j) acc[j] = 0.0f;

    if (col < N) {
        for (int64_t r0 = r_begin + slot * kRows; r0 < r_end; r0 += SLOTS * kRows) {
            const int nr = (int)min((int64_t)kRows, r_end - r0);
            if (nr == kRows) {
                u32x4_t w[kRows];
#pragma unroll
                for (int r = 0; r < kRows; ++r)
                    w[r] = load_row16<ALIGNED>(Q, (r0 + r) * ldq + col, total);
                __builtin_amdgcn_sched_barrier(0);  // all rows in flight first
#pragma unroll
                for (int r = 0; r < kRows; ++r) {
                    const float xr = xs[r0 + r - r_begin];
                    fma_i8_word(xr, w[r].x, acc + 0);
                    fma_i8_word(xr, w[r].y, acc + 4);
                    fma_i8_word(xr, w[r].z, acc + 8);
                    fma_i8_word(xr, w[r].w, acc + 12);
                }
            } else {
                for (int r = 0; r < nr; ++r) {
                    const u32x4_t w = load_row16<ALIGNED>(Q, (r0 + r) * ldq + col, total);
                    const float xr = xs[r0 + r - r_begin];
                    fma_i8_word(xr, w.x, acc + 0);
                    fma_i8_word(xr, w.y, acc + 4);
                    fma_i8_word(xr, w.z, acc + 8);
                    fma_i8_word(xr, w.w, acc + 12);
                }
            }
        }
    }

#pragma unroll
    for (int j = 0; j < kLaneCols; ++j) red[slot * kTN + j * 16 + li] = acc[j];
    __syncthreads();

    for (int c = tid; c < kTN; c += 64 * WAVES) {
        const int ci = (c & 15) * 16 + (c >> 4);
        float v = 0.0f;
#pragma unroll
        for (int s = 0; s < SLOTS; ++s) v += red[s * kTN + ci];
        const int64_t n = tile * kTN + c;
        if (splits == 1) {
            if (n < N) logits[n] = (v * 16777216.0f) * hs[n];
        } else {
            part[split * npad + n] = v;
        }
    }
}

// One launch, no partial sums: a workgroup of WV waves owns 16 LPR columns
// and all K = L WV 64 / LPR rows.  Lane (r, j) = (lane / LPR, lane % LPR) of
// wave w takes the L consecutive rows k = (w 64 / LPR + r) L + i and, of
// each, the 16 bytes of columns n0 + 16 j .. n0 + 16 j + 15, so the LPR lanes
// of a row read 16 LPR contiguous bytes (with LPR = 8 one cache line) and a
// load instruction covers 64 / LPR rows.  Every row's load is issued before
// the first product.  The 16 column sums of a lane are added over the wave's
// row lanes by a fixed xor butterfly (every lane ends with the same totals),
// then over the waves in wave order in LDS.
template <int L, bool ALIGNED, int LPR, int WV>
__global__ __launch_bounds__(64 * WV) void k_head_whole(const float *__restrict__ x, int K,
                                                        const int8_t *__restrict__ Q, int64_t ldq,
                                                        const float *__restrict__ hs, int N,
                                                        float *__restrict__ logits) {
    constexpr int CW = 16 * LPR, RPI = 64 / LPR;  // columns per workgroup, rows per instruction
    __shared__ float red[WV][CW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane / LPR, j = lane % LPR;
    const int n0 = blockIdx.x * CW;
    const int col = n0 + 16 * j;
    // a chunk wholly past N re-reads the last chunk holding column N - 1
    const int cc = col < N ? col : ((N - 1) & ~15);
    const int k0 = (RPI * wave + r) * L;
    const int64_t total = (int64_t)K * ldq;

    float xr[L];
#pragma unroll
    for (int i = 0; i < L; ++i) xr[i] = x[k0 + i];
    u32x4_t w[L];
#pragma unroll
    for (int i = 0; i < L; ++i) w[i] = load_row16<ALIGNED>(Q, (int64_t)(k0 + i) * ldq + cc, total);
    __builtin_amdgcn_sched_barrier(0);  // every row in flight first

    float acc[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] = 0.0f;
#pragma unroll
    for (int i = 0; i < L; ++i) {
        fma_i8_word(xr[i], w[i].x, acc + 0);
        fma_i8_word(xr[i], w[i].y, acc + 4);
        fma_i8_word(xr[i], w[i].z, acc + 8);
        fma_i8_word(xr[i], w[i].w, acc + 12);
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        float v = acc[c];
#pragma unroll
        for (int m = LPR; m < 64; m *= 2) v += __shfl_xor(v, m);
        acc[c] = v;
    }
    if (r == 0) {
#pragma unroll
        for (int c = 0; c < 16; ++c) red[wave][16 * j + c] = acc[c];
    }
    __syncthreads();
    for (int t = tid; t < CW; t += 64 * WV) {
        const int n = n0 + t;
        float v = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < WV; ++w2) v += red[w2][t];
        if (n < N) logits[n] = (v * 16777216.0f) * hs[n];
    }
}

}  // namespace

hipError_t launch_head_quantize(const float *E, int64_t K, int64_t N, int64_t ldq, int8_t *Q,
                                float *hs, int *d_status, hipStream_t stream) {
    if (ldq == 0) return hipSuccess;
    hipLaunchKernelGGL(k_head_quantize, dim3((unsigned)((ldq + 255) / 256)), dim3(256), 0, stream,
                       E, K, N, ldq, Q, hs, d_status);
    return hipGetLastError();
}

hipError_t launch_embed(const int64_t *tokens, int64_t T, const int8_t *Q, int64_t ldq,
                        const float *hs, int64_t K, int64_t N, float *out, int *d_status,
                        hipStream_t stream) {
    const int64_t total = T * K;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_embed, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       tokens, T, Q, ldq, hs, K, N, out, d_status);
    return hipGetLastError();
}

hipError_t launch_head_logits(const HeadPlan &p, const float *x, int64_t K, const int8_t *Q,
                              int64_t ldq, const float *hs, int64_t N, float *logits,
                              void *workspace, hipStream_t stream) {
    if (p.kind == HeadPlan::kEmpty) return hipSuccess;
    if (p.kind == HeadPlan::kZero) return launch_bias_fill(nullptr, 1, N, logits, stream);
    if (p.kind == HeadPlan::kWhole) {
        const int cw = 16 * p.lanes_per_row;
        const dim3 grid((unsigned)((N + cw - 1) / cw));
        const bool al = (ldq % 16) == 0;
#define W4_HEAD_WHOLE(LV, LPRV, WVV)                                                            \
    if (p.rows_per_lane == LV && p.lanes_per_row == LPRV && p.waves == WVV) {                   \
        if (al)                                                                                 \
            hipLaunchKernelGGL((k_head_whole<LV, true, LPRV, WVV>), grid, dim3(64 * WVV), 0,      \
                               stream, x, (int)K, Q, ldq, hs, (int)N, logits);                  \
        else                                                                                    \
            hipLaunchKernelGGL((k_head_whole<LV, false, LPRV, WVV>), grid, dim3(64 * WVV), 0,     \
                               stream, x, (int)K, Q, ldq, hs, (int)N, logits);                  \
        return hipGetLastError();                                                               \
    }
        W4_HEAD_WHOLE(4, 16, 16) W4_HEAD_WHOLE(8, 16, 16) W4_HEAD_WHOLE(12, 16, 16)
        W4_HEAD_WHOLE(16, 16, 16)
        W4_HEAD_WHOLE(4, 8, 8) W4_HEAD_WHOLE(8, 8, 8) W4_HEAD_WHOLE(12, 8, 8) W4_HEAD_WHOLE(16, 8, 8)
#undef W4_HEAD_WHOLE
        return hipErrorInvalidValue;
    }
    float *part = p.splits > 1 ? static_cast<float *>(workspace) : nullptr;
    const dim3 grid((unsigned)(p.tiles * p.splits));
    const bool aligned = (ldq % 16) == 0;
    const size_t shm = (size_t)(p.waves * kGemvGroups * kTN + p.rows_per_wg) * sizeof(float);
#define W4_HEAD_CASE(WV)                                                                        \
    case WV:                                                                                    \
        if (aligned)                                                                            \
            hipLaunchKernelGGL((k_head_logits<WV, true>), grid, dim3(64 * WV), shm, stream, x, K,  \
                               Q, ldq, hs, N, logits, p.tiles, p.splits, p.rows_per_wg, p.npad,  \
                               part);                                                           \
        else                                                                                    \
            hipLaunchKernelGGL((k_head_logits<WV, false>), grid, dim3(64 * WV), shm, stream, x, K, \
                               Q, ldq, hs, N, logits, p.tiles, p.splits, p.rows_per_wg, p.npad,  \
                               part);                                                           \
        break;
    switch (p.waves) {
        W4_HEAD_CASE(1)
        W4_HEAD_CASE(2)
        W4_HEAD_CASE(4)
    default:
        return hipErrorInvalidValue;
    }
#undef W4_HEAD_CASE
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_reduce(part, p.splits, 1, N, p.npad, nullptr, hs, 16777216.0f, logits,
                                stream);
}

}  // namespace w4
