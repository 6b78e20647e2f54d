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
// Head on the integer matrix cores.  The table codes are exact int8, so they
// are the B operand of v_mfma_i32_16x16x64_i8 as loaded: no conversion at
// all.  The activation row x (fp32) is written as a 31-bit fixed-point number
// relative to 2^e, where e is the exponent of max|x|:
//   v_k = rint(x_k * 2^(30-e)),  |v_k| <= 2^30,  |x_k - v_k 2^(e-30)| <= 2^(e-31)
// and split into four signed 8-bit digits v = L0 + 2^8 L1 + 2^16 L2 + 2^24 L3,
// which are rows 0-3 of the A operand.  The MFMAs accumulate sum_k L_i[k] Q[k,n]
// exactly in int32 (|sum| < 2^31 for K <= 8192), and the four row sums are
// combined exactly in fp64, so the only rounding is that of x to fixed point
// (at most 2^-30 max|x| per element) and the final scaling by hs[n] 2^(e-30).
// Non-finite x gives NaN logits.
#include <limits.h>

#include "common.h"
#include "launch.h"

namespace w4 {
namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

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

// One wave: 16 columns (tokens) n0 .. n0+15 over all of K, in chunks of CH
// MFMAs of 64 k each.  Lane (g, c) = (lane / 16, lane % 16): B is the 16
// bytes Qt[n0 + c, 64 j + 16 g ...], A is limb row c (c < 4) of the same 16 k.
// The four waves of a workgroup take adjacent 16-column tiles and share the
// limbs of x, built once per workgroup in LDS.
template <int CH, int XPT, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_head_logits_mfma(const float *__restrict__ x, int K,
                                                          const int8_t *__restrict__ Qt, int ldt,
                                                          const float *__restrict__ hs, int N,
                                                          float *__restrict__ logits) {
    extern __shared__ i32x4_t limbs_v[];  // [4][K] bytes, 16-byte aligned
    int8_t *limbs = reinterpret_cast<int8_t *>(limbs_v);
    __shared__ float wmax[WAVES];
    constexpr int T = 64 * WAVES;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int nbase = blockIdx.x * (16 * WAVES) + wave * 16;
    const int n = min(nbase + c, N - 1);  // past N: re-read the last row, store nothing
    const int NJ = K / 64;

    // x first (the loads the prologue waits for), then this lane's first chunk
    // of table rows, so the table stream starts before the prologue's barriers
    float xv[XPT];  // XPT * T >= K; loads clamped, values past K zeroed
#pragma unroll
    for (int i = 0; i < XPT; ++i) xv[i] = x[min(tid + T * i, K - 1)];
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t rowoff = (uint32_t)n * (uint32_t)ldt + 16u * g;
    u32x4_t b[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j)
        b[j] = load_stream<u32x4_t>(Qt + rowoff + 64u * (uint32_t)min(j, NJ - 1));
    __builtin_amdgcn_sched_barrier(0);  // every load issued before any use of x
#pragma unroll
    for (int i = 0; i < XPT; ++i)
        if (tid + T * i >= K) xv[i] = 0.0f;

    // max |x| over the workgroup (every workgroup computes the same value)
    float m = 0.0f;
    bool finite = true;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        finite &= __builtin_isfinite(xv[i]);
        m = __builtin_fmaxf(m, __builtin_fabsf(xv[i]));
    }
    if (!finite) m = __builtin_inff();
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o));
    if (WAVES > 1) {
        if (lane == 0) wmax[wave] = m;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < WAVES; ++w) m = __builtin_fmaxf(m, wmax[w]);
    }
    const float amax = m;
    const bool ok = __builtin_isfinite(amax);
    int e = 0;
    if (ok && amax > 0.0f) (void)__builtin_frexpf(amax, &e);  // amax < 2^e
    // digits of v = rint(x * 2^(30 - e)), written as limbs[i][k]
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int k = tid + T * i;
        if (k < K) {
            const int v = ok ? (int)__builtin_rintf(__builtin_ldexpf(xv[i], 30 - e)) : 0;
            const int l0 = (int)(int8_t)(v & 0xFF);
            const int v1 = (v - l0) >> 8;
            const int l1 = (int)(int8_t)(v1 & 0xFF);
            const int v2 = (v1 - l1) >> 8;
            const int l2 = (int)(int8_t)(v2 & 0xFF);
            const int l3 = (v2 - l2) >> 8;  // |l3| <= 64
            limbs[k] = (int8_t)l0;
            limbs[K + k] = (int8_t)l1;
            limbs[2 * K + k] = (int8_t)l2;
            limbs[3 * K + k] = (int8_t)l3;
        }
    }
    __syncthreads();

    i32x4_t acc = {0, 0, 0, 0};
    const i32x4_t zero = {0, 0, 0, 0};
    for (int j0 = 0; j0 < NJ; j0 += CH) {
        if (j0 > 0) {
#pragma unroll
            for (int j = 0; j < CH; ++j)
                b[j] = load_stream<u32x4_t>(Qt + rowoff + 64u * (uint32_t)min(j0 + j, NJ - 1));
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int jj = j0 + j;
            i32x4_t a = zero;
            if (c < 4 && jj < NJ)
                a = *reinterpret_cast<const i32x4_t *>(limbs + c * K + 64 * jj + 16 * g);
            if (jj < NJ)
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                    a, __builtin_bit_cast(i32x4_t, b[j]), acc, 0, 0, 0);
        }
    }

    // lanes 0-15 hold D[0..3][c]: the four limb sums of column n0 + c
    if (g == 0 && nbase + c < N) {
        float out;
        if (ok) {
            const double t = ((double)acc[3] * 16777216.0 + (double)acc[2] * 65536.0) +
                             ((double)acc[1] * 256.0 + (double)acc[0]);
            out = (float)(__builtin_ldexp(t, e - 30) * (double)hs[n]);
        } else {
            out = __builtin_nanf("");
        }
        logits[nbase + c] = out;
    }
}

// Full-sequence logits, first launch: the digit image of x, built once.
// One workgroup per group of 4 rows.  A-operand row a = 4 r + l of the group
// is digit l of row r (each row has its own exponent e_r), laid out in the
// order the MFMA lanes read it: per K-step j one 1 KB block of 64 16-byte
// elements, element 16 h + a holding the digits of x[4 group + r,
// 64 j + 16 h .. 64 j + 16 h + 15] (lane l = 16 h + a reads element l, so a
// wave's read is one contiguous kilobyte, free of LDS bank conflicts).
// erow[m] is e_m, or INT_MIN for a row with a non-finite entry.  Rows past M
// are zero.
template <int XPT>
__global__ __launch_bounds__(256) void k_head_digits(const float *__restrict__ x, int M, int K,
                                                     int8_t *__restrict__ img,
                                                     int *__restrict__ erow) {
    extern __shared__ i32x4_t dimg_v[];  // [K / 64][16][64] bytes
    int8_t *dimg = reinterpret_cast<int8_t *>(dimg_v);
    __shared__ float wmax[4][4];
    const int m0 = 4 * blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int RK = 4 * K;

    float xv[XPT];  // element e = tid + 256 i of the 4 x K block
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int e = tid + 256 * i;
        const int r = e / K;
        xv[i] = (e < RK && m0 + r < M) ? x[(size_t)(m0 + r) * K + (e - r * K)] : 0.0f;
    }
    // per-row max |x| (a non-finite entry makes its row's max infinite)
    float mr[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int r = (tid + 256 * i) / K;
        const float a = __builtin_isfinite(xv[i]) ? __builtin_fabsf(xv[i]) : __builtin_inff();
#pragma unroll
        for (int q = 0; q < 4; ++q) mr[q] = (r == q) ? __builtin_fmaxf(mr[q], a) : mr[q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mr[q] = __builtin_fmaxf(mr[q], __shfl_xor(mr[q], o));
        if (lane == 0) wmax[wave][q] = mr[q];
    }
    __syncthreads();
    int er[4];
    bool okr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float am = __builtin_fmaxf(__builtin_fmaxf(wmax[0][q], wmax[1][q]),
                                         __builtin_fmaxf(wmax[2][q], wmax[3][q]));
        okr[q] = __builtin_isfinite(am);
        er[q] = 0;
        if (okr[q] && am > 0.0f) (void)__builtin_frexpf(am, &er[q]);
    }
    if (tid < 4 && m0 + tid < M) {
        int e = er[0];
        bool ok = okr[0];
#pragma unroll
        for (int q = 1; q < 4; ++q)
            if (tid == q) {
                e = er[q];
                ok = okr[q];
            }
        erow[m0 + tid] = ok ? e : INT_MIN;
    }
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int e = tid + 256 * i;
        if (e < RK) {
            const int r = e / K, k = e - r * K;
            int eq = er[0];
            bool oq = okr[0];
#pragma unroll
            for (int q = 1; q < 4; ++q)
                if (r == q) {
                    eq = er[q];
                    oq = okr[q];
                }
            const int v = oq ? (int)__builtin_rintf(__builtin_ldexpf(xv[i], 30 - eq)) : 0;
            const int l0 = (int)(int8_t)(v & 0xFF);
            const int v1 = (v - l0) >> 8;
            const int l1 = (int)(int8_t)(v1 & 0xFF);
            const int v2 = (v1 - l1) >> 8;
            const int l2 = (int)(int8_t)(v2 & 0xFF);
            const int l3 = (v2 - l2) >> 8;
            int8_t *d = dimg + (k >> 6) * 1024 + (((k & 63) >> 4) * 16 + 4 * r) * 16 + (k & 15);
            d[0] = (int8_t)l0;
            d[16] = (int8_t)l1;
            d[32] = (int8_t)l2;
            d[48] = (int8_t)l3;
        }
    }
    __syncthreads();
    i32x4_t *dst = reinterpret_cast<i32x4_t *>(img + (size_t)blockIdx.x * 16 * K);
    for (int i = tid; i < K; i += 256) dst[i] = dimg_v[i];  // 16 K bytes
}

// Row groups per LDS chunk: two chunk buffers of at most 32 KB of digit
// blocks each (16 K bytes per group, K >= 64), so at most 32 groups.
constexpr int kHeadRowsMaxChunk = 32;

// Copy `elems` 16-byte elements (a multiple of 64) from global memory to LDS
// with the direct global-to-LDS load: wave w moves elements w*64 + 256 i +
// lane, no registers involved, completion counted by vmcnt.
__device__ __forceinline__ void copy_to_lds(const i32x4_t *__restrict__ src, i32x4_t *dst,
                                            int elems, int wave, int lane) {
    for (int i0 = wave * 64; i0 < elems; i0 += 256)
        __builtin_amdgcn_global_load_lds(static_cast<const void *>(src + i0 + lane),
                                         reinterpret_cast<__attribute__((address_space(3))) void *>(
                                             reinterpret_cast<uintptr_t>(dst + i0)),
                                         16, 0, 0);
}

// Full-sequence logits, second launch: the table stays in registers, the
// rows stream past it.  Wave w of workgroup b owns TB tiles of 16 tokens
// (tokens 16 (TB (4 b + w) + t) + c); it loads their table rows once, as the
// B operands of all K / 64 steps, then takes every row group in turn.  The
// digit blocks come through LDS in chunks of row groups, double-buffered: the
// direct global-to-LDS copy of chunk i + 1 is in flight while the MFMAs run on
// chunk i.  Each A operand read from LDS feeds TB MFMAs, and lane (g, c) ends
// with the four digit sums of row 4 group + g, token c of each tile, combined
// exactly as in the one-row kernel.  The table comes from HBM once; x only
// through the small digit image.
template <int TB, int NJM>
// Arguments: those the prologue needs first, within the 14 preloaded
// argument registers; the logits pointer last.
__global__ __launch_bounds__(256) void k_head_rows_mfma(const int8_t *__restrict__ img,
                                                        const int *__restrict__ erow,
                                                        const int8_t *__restrict__ Qt,
                                                        const float *__restrict__ hs, int M,
                                                        int K, int ldt, int N, int chunk,
                                                        float *__restrict__ logits) {
    extern __shared__ i32x4_t abuf[];  // [2][chunk][K / 64][16][64] bytes
    __shared__ int es[2][kHeadRowsMaxChunk * 4];  // exponents of each buffer's rows
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int NJ = K / 64, nrg = (M + 3) / 4;
    const int tb0 = (blockIdx.x * 4 + wave) * 16 * TB;
    const int per_rg = NJ * 64;  // 16-byte elements per row group
    i32x4_t *bufs[2] = {abuf, abuf + chunk * per_rg};
    const i32x4_t *src = reinterpret_cast<const i32x4_t *>(img);

    // stage one chunk (rows 4 rg0 ...) into buffer q: digit blocks and exponents
    auto stage = [&](int rg0, int q) {
        const int cnt = min(chunk, nrg - rg0);
        copy_to_lds(src + (size_t)rg0 * per_rg, bufs[q], cnt * per_rg, wave, lane);
        if (wave == 0 && lane < 4 * cnt && 4 * rg0 + lane < M)
            __builtin_amdgcn_global_load_lds(
                static_cast<const void *>(erow + 4 * rg0 + lane),
                reinterpret_cast<__attribute__((address_space(3))) void *>(
                    reinterpret_cast<uintptr_t>(&es[q][0])),
                4, 0, 0);
    };

    stage(0, 0);
    u32x4_t b[TB][NJM];
    float hsv[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        const int n = min(tb0 + 16 * t + c, N - 1);
        const uint32_t rowoff = (uint32_t)n * (uint32_t)ldt + 16u * g;
#pragma unroll
        for (int j = 0; j < NJM; ++j)
            b[t][j] = load_stream<u32x4_t>(Qt + rowoff + 64u * (uint32_t)min(j, NJ - 1));
        hsv[t] = hs[n];
    }

    int q = 0;
    for (int rg0 = 0; rg0 < nrg; rg0 += chunk, q ^= 1) {
        const int cnt = min(chunk, nrg - rg0);
        // this chunk's copies (and the table rows) have landed, in every wave;
        // every wave is also done with the other buffer (read last round)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (rg0 + chunk < nrg) stage(rg0 + chunk, q ^ 1);
        const i32x4_t *cb = bufs[q];
        for (int r = 0; r < cnt; ++r) {
            // two accumulators per tile (even and odd K-steps): twice as many
            // independent MFMA chains; int32 sums, so the order is exact
            i32x4_t acc2[2][TB];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int t = 0; t < TB; ++t) acc2[h][t] = i32x4_t{0, 0, 0, 0};
            // straight-line: steps past K read a valid block and multiply a
            // zero A operand (adds exactly 0), so the LDS reads can be issued
            // ahead of the MFMAs; when K fills every step no select is needed
            const i32x4_t *ap = cb + r * per_rg + lane;
            i32x4_t a[NJM];
#pragma unroll
            for (int j = 0; j < NJM; ++j) a[j] = ap[min(j, NJ - 1) * 64];
            if (NJ == NJM) {
#pragma unroll
                for (int j = 0; j < NJM; ++j)
#pragma unroll
                    for (int t = 0; t < TB; ++t)
                        acc2[j & 1][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                            a[j], __builtin_bit_cast(i32x4_t, b[t][j]), acc2[j & 1][t], 0, 0, 0);
            } else {
#pragma unroll
                for (int j = 0; j < NJM; ++j) {
                    const i32x4_t aj = j < NJ ? a[j] : i32x4_t{0, 0, 0, 0};
#pragma unroll
                    for (int t = 0; t < TB; ++t)
                        acc2[j & 1][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                            aj, __builtin_bit_cast(i32x4_t, b[t][j]), acc2[j & 1][t], 0, 0, 0);
                }
            }
            i32x4_t acc[TB];
#pragma unroll
            for (int t = 0; t < TB; ++t) acc[t] = acc2[0][t] + acc2[1][t];
            const int m = 4 * (rg0 + r) + g;
            if (m < M) {
                const int e = es[q][4 * r + g];
#pragma unroll
                for (int t = 0; t < TB; ++t) {
                    const int n = tb0 + 16 * t + c;
                    if (n < N) {
                        float out = __builtin_nanf("");
                        if (e != INT_MIN) {
                            const double v = ((double)acc[t][3] * 16777216.0 +
                                              (double)acc[t][2] * 65536.0) +
                                             ((double)acc[t][1] * 256.0 + (double)acc[t][0]);
                            out = (float)(__builtin_ldexp(v, e - 30) * (double)hsv[t]);
                        }
                        logits[(size_t)m * N + n] = out;
                    }
                }
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

hipError_t launch_head_logits_kmajor(const float *x, int64_t K, const int8_t *Qt, int64_t ldt,
                                     const float *hs, int64_t N, float *logits,
                                     hipStream_t stream) {
    const size_t shm = (size_t)4 * K;
    const int waves = plan_head_kmajor_waves(K, N);
    const dim3 gridw((unsigned)((N + 16 * waves - 1) / (16 * waves)));
#define W4_HK(CHV, XV, WV)                                                                         \
    hipLaunchKernelGGL((k_head_logits_mfma<CHV, XV, WV>), gridw, dim3(64 * WV), shm, stream, x,   \
                       (int)K, Qt, (int)ldt, hs, (int)N, logits)
#define W4_HK3(CHV)                                                                               \
    if (waves == 1) W4_HK(CHV, CHV, 1);                                                           \
    else if (waves == 2) W4_HK(CHV, CHV / 2, 2);                                                  \
    else W4_HK(CHV, CHV / 4, 4);
    if (K <= 256) { W4_HK3(4) }
    else if (K <= 512) { W4_HK3(8) }
    else if (K <= 768) { W4_HK3(12) }
    else if (K <= 1024) { W4_HK3(16) }
    else W4_HK(16, 32, 4);
#undef W4_HK3
#undef W4_HK
    return hipGetLastError();
}

size_t head_rows_workspace(int64_t M, int64_t K) {
    const int64_t nrg = (M + 3) / 4;
    const size_t img = ((size_t)nrg * 16 * K + 255) / 256 * 256;
    return img + (size_t)4 * M;
}

hipError_t launch_head_rows_kmajor(const float *x, int64_t M, int64_t K, const int8_t *Qt,
                                  int64_t ldt, const float *hs, int64_t N, float *logits,
                                  void *workspace, hipStream_t stream) {
    const int64_t nrg = (M + 3) / 4;
    int8_t *img = static_cast<int8_t *>(workspace);
    int *erow = reinterpret_cast<int *>(img + (head_rows_workspace(M, K) - (size_t)4 * M));
    const size_t dshm = (size_t)16 * K;
#define W4_HD(XV)                                                                                 \
    hipLaunchKernelGGL((k_head_digits<XV>), dim3((unsigned)nrg), dim3(256), dshm, stream, x,      \
                       (int)M, (int)K, img, erow)
    if (K <= 256) W4_HD(4);
    else if (K <= 512) W4_HD(8);
    else if (K <= 1024) W4_HD(16);
    else W4_HD(32);
#undef W4_HD
    // two LDS buffers of a chunk of row groups each, at most 32 KB per buffer
    // (64 KB per workgroup, so two workgroups fit a compute unit)
    const int64_t per_rg = (int64_t)16 * K;
    int64_t chunk = ((int64_t)32 << 10) / per_rg;
    if (chunk < 1) chunk = 1;
    if (chunk > kHeadRowsMaxChunk) chunk = kHeadRowsMaxChunk;
    if (chunk > nrg) chunk = nrg;
    const size_t shm = (size_t)(2 * chunk * per_rg);
#define W4_HR(TBV, NJV)                                                                           \
    hipLaunchKernelGGL((k_head_rows_mfma<TBV, NJV>),                                             \
                       dim3((unsigned)((N + 64 * TBV - 1) / (64 * TBV))), dim3(256), shm, stream, \
                       img, erow, Qt, hs, (int)M, (int)K, (int)ldt, (int)N, (int)chunk, logits)
    if (K <= 256) W4_HR(2, 4);
    else if (K <= 512) W4_HR(2, 8);
    else if (K <= 768) W4_HR(2, 12);
    else if (K <= 1024) W4_HR(2, 16);
    else W4_HR(1, 32);
#undef W4_HR
    return hipGetLastError();
}

}  // namespace w4
