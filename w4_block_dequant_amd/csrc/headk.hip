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

// Full-sequence logits: 4 rows of x per workgroup.  A-operand row 4 r + l is
// digit l of row r (each row has its own exponent e_r), so all 16 rows of the
// MFMA carry data and lane (g, c) ends with the four digit sums of row g,
// column c.  The table is the same B operand as above.  Workgroups that share
// a 64-token tile (one per group of 4 rows) are given ids that map to the same
// XCD (ids are dealt to the 8 XCDs in turn), so the tile's table rows come
// from HBM about once and from that XCD's L2 for the other row groups.
template <int CH, int XPT>
__global__ __launch_bounds__(256) void k_head_rows_mfma(const float *__restrict__ x, int M, int K,
                                                        const int8_t *__restrict__ Qt, int ldt,
                                                        const float *__restrict__ hs, int N,
                                                        float *__restrict__ logits, int ntiles,
                                                        int nrg) {
    extern __shared__ i32x4_t limbs_v[];  // [16][K] bytes: row 4 r + l = digit l of row r
    int8_t *limbs = reinterpret_cast<int8_t *>(limbs_v);
    __shared__ float wmax[4][4];
    const int id = blockIdx.x, xcd = id & 7, local = id >> 3;
    const int tile = (local / nrg) * 8 + xcd, rg = local % nrg;
    if (tile >= ntiles) return;  // whole workgroup, before any barrier
    const int m0 = 4 * rg;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int nbase = tile * 64 + wave * 16;
    const int n = min(nbase + c, N - 1);
    const int NJ = K / 64, RK = 4 * K;

    // x of the 4 rows first, then the table rows (as in the 1-row kernel)
    float xv[XPT];  // element e = tid + 256 i of the 4 x K block
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int e = min(tid + 256 * i, RK - 1);
        const int r = e / K;
        xv[i] = x[(size_t)min(m0 + r, M - 1) * K + (e - r * K)];
    }
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t rowoff = (uint32_t)n * (uint32_t)ldt + 16u * g;
    u32x4_t b[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j)
        b[j] = load_stream<u32x4_t>(Qt + rowoff + 64u * (uint32_t)min(j, NJ - 1));
    __builtin_amdgcn_sched_barrier(0);

    // per-row max |x| (a non-finite entry makes its row's max infinite)
    float mr[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int e = tid + 256 * i;
        const int r = e / K;
        const bool valid = e < RK && m0 + r < M;
        if (!valid) xv[i] = 0.0f;
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
            int8_t *lr = limbs + (4 * r) * K + k;
            lr[0] = (int8_t)l0;
            lr[K] = (int8_t)l1;
            lr[2 * K] = (int8_t)l2;
            lr[3 * K] = (int8_t)l3;
        }
    }
    __syncthreads();

    i32x4_t acc = {0, 0, 0, 0};
    for (int j0 = 0; j0 < NJ; j0 += CH) {
        if (j0 > 0) {
#pragma unroll
            for (int j = 0; j < CH; ++j)
                b[j] = load_stream<u32x4_t>(Qt + rowoff + 64u * (uint32_t)min(j0 + j, NJ - 1));
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int jj = j0 + j;
            if (jj < NJ) {
                const i32x4_t a =
                    *reinterpret_cast<const i32x4_t *>(limbs + c * K + 64 * jj + 16 * g);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                    a, __builtin_bit_cast(i32x4_t, b[j]), acc, 0, 0, 0);
            }
        }
    }

    // lane (g, c) holds the four digit sums of row m0 + g, column nbase + c
    const int m = m0 + g;
    if (m < M && nbase + c < N) {
        int eg = er[0];
        bool og = okr[0];
#pragma unroll
        for (int q = 1; q < 4; ++q)
            if (g == q) {
                eg = er[q];
                og = okr[q];
            }
        float out = __builtin_nanf("");
        if (og) {
            const double t = ((double)acc[3] * 16777216.0 + (double)acc[2] * 65536.0) +
                             ((double)acc[1] * 256.0 + (double)acc[0]);
            out = (float)(__builtin_ldexp(t, eg - 30) * (double)hs[n]);
        }
        logits[(size_t)m * N + nbase + c] = out;
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

hipError_t launch_head_rows_kmajor(const float *x, int64_t M, int64_t K, const int8_t *Qt,
                                  int64_t ldt, const float *hs, int64_t N, float *logits,
                                  hipStream_t stream) {
    const int ntiles = (int)((N + 63) / 64), nrg = (int)((M + 3) / 4);
    const int64_t wgs = (int64_t)((ntiles + 7) / 8) * 8 * nrg;
    const size_t shm = (size_t)16 * K;
#define W4_HR(CHV, XV)                                                                            \
    hipLaunchKernelGGL((k_head_rows_mfma<CHV, XV>), dim3((unsigned)wgs), dim3(256), shm, stream, x, \
                       (int)M, (int)K, Qt, (int)ldt, hs, (int)N, logits, ntiles, nrg)
    if (K <= 256) W4_HR(4, 4);
    else if (K <= 512) W4_HR(8, 8);
    else if (K <= 768) W4_HR(12, 12);
    else if (K <= 1024) W4_HR(16, 16);
    else W4_HR(16, 32);
#undef W4_HR
    return hipGetLastError();
}

}  // namespace w4
