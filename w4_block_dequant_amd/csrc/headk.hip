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

// Full-sequence logits on the bf16 matrix cores with exact operands (M >= 4,
// K <= 1024).  A token's codes are exact in bf16 (|Q| <= 127), and every fp32
// activation is exactly h + m + l with h = bf16(x), m = bf16(x - h),
// l = x - h - m (each difference exact in fp32, l exact in bf16), so each
// v_mfma_f32_16x16x32_bf16 forms exact products and only its fp32
// accumulation rounds, as in the fp32 kernel; hs[n] is applied at the end.
//
// One wave owns 16 TT tokens (lane c = lane % 16 is token t0 + 16 tt + c of
// token tile tt) for all rows; a workgroup of WAVES waves shares each row
// tile's activation parts.  With TT = 2 every A read from LDS feeds the MFMAs
// of both token tiles (half the LDS traffic per product); the codes then stay
// in registers as the int8 bytes they are and are widened to bf16 per step.
// Lane group g = lane / 16 owns bytes 16 g .. 16 g + 15 of every 64-byte piece
// of the padded K (KP, a multiple of 64), 8 k per MFMA step: its codes
// come in whole 16-byte loads, are turned into bf16 once and stay in
// registers (4 dwords per step).  The rows pass through LDS one 16-row tile
// at a time as three bf16 part planes [part][row][KP + 8] (the 8-element pad
// spreads the rows over the LDS banks), built once per workgroup; the A
// operand of step s for lane (g, r) is row r's parts at k = 64 (s / 2) +
// 16 g + 8 (s % 2).  So a code load instruction reads 64 contiguous bytes of
// each of 16 token rows (a lane group's quarter of K in one run would touch
// 64 cache lines per instruction instead).
// Rows with a non-finite entry are flagged while they are built and give NaN.
// With two token tiles (K <= 768) each row tile's activations reach LDS as
// they are, by direct-to-LDS loads (global_load_lds_dwordx4: a wave writes
// 1 KB of consecutive LDS per instruction, no registers) into a second
// buffer [16][K] fp32 after the part planes: the first tile's before the
// codes are loaded, each later tile's while the previous tile's MFMAs run;
// the barriers fence LDS only, and a tile's logits are stored after the next
// tile's wait.  That wait (vmcnt also counts stores) would otherwise drain
// the stores just issued, and a full workgroup fence, or activation loads
// queued behind the codes, would hold every build behind the code stream.
template <int SMAX, int WAVES, int TT>
__global__ __launch_bounds__(64 * WAVES) void k_head_rows_x3(const float *__restrict__ x, int M, int K,
                                                      const int8_t *__restrict__ Qt, int ldt,
                                                      const float *__restrict__ hs, int N,
                                                      float *__restrict__ logits) {
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    extern __shared__ u32x4_t aplane_v[];  // [3][16][KP + 8] bf16
    __shared__ int rowbad[16];
    uint16_t *ap = reinterpret_cast<uint16_t *>(aplane_v);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int t0 = (blockIdx.x * WAVES + wave) * 16 * TT;
    const int KP = (K + 63) / 64 * 64, S = KP / 32, RS = KP + 8;
    const int n = min(t0 + c, N - 1);

    // TT = 2: raw activations of a row tile, [16][K] fp32 after the planes
    constexpr bool DMA = TT == 2;
    float *xr = reinterpret_cast<float *>(ap + 3 * 16 * RS);
    // rows m0 .. m0 + 15 of x (those below M) to xr: 1 KB chunk j of the
    // tile (16 K floats, contiguous in x) by wave j % WAVES, lane l taking
    // bytes 16 l of the chunk
    const int tile_chunks = (16 * K * 4 + 1023) / 1024;
    auto dma_tile = [&](int m0) {
        const int valid = min(16, M - m0) * K * 4;  // bytes of the tile inside x
        const char *src0 = reinterpret_cast<const char *>(x + (size_t)m0 * K);
        for (int j = wave; j < tile_chunks; j += WAVES) {
            const int off = 1024 * j + 16 * lane;
            if (off < valid)
                __builtin_amdgcn_global_load_lds(
                    src0 + off,
                    (__attribute__((address_space(3))) void *)(reinterpret_cast<char *>(xr) + 1024 * j),
                    16, 0, 0);
        }
    };
    auto lds_barrier = []() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };
    if (DMA) {
        dma_tile(0);
        __builtin_amdgcn_sched_barrier(0);
    }
    // DMA: the previous tile's logits (scaled), its row flags and first row
    float pend[TT][4];
    uint32_t pbad = 0;
    int pm0 = -1;
    auto store_pending = [&]() {
        if (pm0 < 0) return;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const int t = t0 + 16 * tt + c;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = pm0 + 4 * g + v;
                if (m < M && t < N)
                    logits[(size_t)m * N + t] = ((pbad >> v) & 1) ? __builtin_nanf("") : pend[tt][v];
            }
        }
    };

    // TT = 2: the codes of both token tiles as loaded, 16 bytes per two steps
    // (the compiler widens them to bf16 once, outside the row-tile loop)
    u32x4_t qb[TT == 2 ? 2 : 1][TT == 2 ? SMAX / 2 : 1];
    float hsn2[2] = {0.0f, 0.0f};
    if (TT == 2) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int nt = min(t0 + 16 * tt + c, N - 1);
            const int8_t *row = Qt + (size_t)nt * ldt;
#pragma unroll
            for (int j = 0; j < SMAX / 2; ++j)
                if (2 * j < S)
                    qb[tt][j] = *reinterpret_cast<const u32x4_t *>(row + min(64 * j + 16 * g, ldt - 16));
            hsn2[tt] = hs[nt];
        }
    }
    // TT = 1: codes of this lane's token and k range, as bf16 pairs: step s uses b[s]
    u32x4_t b[TT == 1 ? SMAX : 1];
    if (TT == 1) {
        const int8_t *row = Qt + (size_t)n * ldt;
#pragma unroll
        for (int j = 0; j < SMAX / 2; ++j) {
            if (2 * j < S) {
                const int k0 = min(64 * j + 16 * g, ldt - 16);  // past K: a valid piece, zero A
                // ordinary (cached) loads: a load instruction covers 64
                // contiguous bytes of each of 16 rows
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(row + k0);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
                uint32_t o[8];
#pragma unroll
                for (int d = 0; d < 4; ++d)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const float lo = (float)(int)(int8_t)(w[d] >> (16 * h));
                        const float hi = (float)(int)(int8_t)(w[d] >> (16 * h + 8));
                        // bf16 of a small integer is the upper half of its fp32 bits
                        o[2 * d + h] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi),
                                                             __builtin_bit_cast(uint32_t, lo),
                                                             0x07060302u);
                    }
                b[2 * j] = u32x4_t{o[0], o[1], o[2], o[3]};
                b[2 * j + 1] = u32x4_t{o[4], o[5], o[6], o[7]};
            }
        }
    }
    const float hsn = TT == 1 ? hs[n] : 0.0f;
    // 8 int8 codes (two dwords) as four bf16 pairs
    auto widen = [](uint32_t w0, uint32_t w1) {
        const uint32_t w[2] = {w0, w1};
        uint32_t o[4];
#pragma unroll
        for (int d = 0; d < 2; ++d)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float lo = (float)(int)(int8_t)(w[d] >> (16 * h));
                const float hi = (float)(int)(int8_t)(w[d] >> (16 * h + 8));
                o[2 * d + h] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi),
                                                     __builtin_bit_cast(uint32_t, lo), 0x07060302u);
            }
        return u32x4_t{o[0], o[1], o[2], o[3]};
    };
    const int K8 = KP / 8;  // 8-element pieces per row

    for (int m0 = 0; m0 < M; m0 += 16) {
        if (DMA) {
            // this wave's chunks of the tile are in LDS (and every load and
            // store it issued before them is done); the barriers make every
            // wave's chunks visible and end the previous tile's reads
            __builtin_amdgcn_s_waitcnt(0);
            lds_barrier();
            store_pending();
            if (tid < 16) rowbad[tid] = 0;
            lds_barrier();
        } else {
            __syncthreads();  // the previous tile's reads are done
            if (tid < 16) rowbad[tid] = 0;
            __syncthreads();
        }
        // build: piece e = (row, 8 k) of the tile, three bf16 parts each
        for (int e = tid; e < 16 * K8; e += 64 * WAVES) {
            const int r = e / K8, k = 8 * (e - r * K8);
            float xv[8];
            const bool live = m0 + r < M && k < K;  // K % 16 == 0: a piece is all in or all out
            if (live) {
                const f32x4_t *xp = DMA ? reinterpret_cast<const f32x4_t *>(xr + r * K + k)
                                        : reinterpret_cast<const f32x4_t *>(x + (size_t)(m0 + r) * K + k);
                const f32x4_t a0 = xp[0], a1 = xp[1];
                xv[0] = a0.x; xv[1] = a0.y; xv[2] = a0.z; xv[3] = a0.w;
                xv[4] = a1.x; xv[5] = a1.y; xv[6] = a1.z; xv[7] = a1.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) xv[i] = 0.0f;
            }
            bool fin = true;
            uint32_t ph[4], pm[4], pl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a = xv[2 * i], bq = xv[2 * i + 1];
                fin &= __builtin_isfinite(a) && __builtin_isfinite(bq);
                const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, bq}, bf16x2_t));
                const float ra = a - __builtin_bit_cast(float, h << 16);
                const float rb = bq - __builtin_bit_cast(float, h & 0xFFFF0000u);
                const uint32_t m = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{ra, rb}, bf16x2_t));
                const float la = ra - __builtin_bit_cast(float, m << 16);
                const float lb = rb - __builtin_bit_cast(float, m & 0xFFFF0000u);
                ph[i] = h;
                pm[i] = m;
                pl[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{la, lb}, bf16x2_t));
            }
            if (!fin) rowbad[r] = 1;
            *reinterpret_cast<u32x4_t *>(ap + (0 * 16 + r) * RS + k) = u32x4_t{ph[0], ph[1], ph[2], ph[3]};
            *reinterpret_cast<u32x4_t *>(ap + (1 * 16 + r) * RS + k) = u32x4_t{pm[0], pm[1], pm[2], pm[3]};
            *reinterpret_cast<u32x4_t *>(ap + (2 * 16 + r) * RS + k) = u32x4_t{pl[0], pl[1], pl[2], pl[3]};
        }
        if (DMA) {
            lds_barrier();  // the planes are built and the raw tile is read
            if (m0 + 16 < M) dma_tile(m0 + 16);  // lands while this tile's MFMAs run
        } else {
            __syncthreads();
        }
        // two accumulators per token tile (even and odd steps): independent
        // MFMA chains
        f32x4v acc2[TT][2];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc2[tt][0] = acc2[tt][1] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < SMAX; ++s) {
            if (s < S) {
                const int k = 64 * (s >> 1) + 16 * g + 8 * (s & 1);
                const bf16x8_t al = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(ap + (2 * 16 + c) * RS + k));
                const bf16x8_t am = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(ap + (1 * 16 + c) * RS + k));
                const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(ap + (0 * 16 + c) * RS + k));
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
                    u32x4_t bw;
                    if (TT == 1) {
                        bw = b[s];
                    } else {
                        const u32x4_t v = qb[tt][s >> 1];
                        bw = (s & 1) ? widen(v.z, v.w) : widen(v.x, v.y);
                    }
                    const bf16x8_t bb = __builtin_bit_cast(bf16x8_t, bw);
                    f32x4v &a = acc2[tt][s & 1];
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bb, a, 0, 0, 0);
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, bb, a, 0, 0, 0);
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bb, a, 0, 0, 0);
                }
            }
        }
        // lane (g, c) holds D[4 g + v][c]: row m0 + 4 g + v, token t0 + 16 tt + c
        if (DMA) {
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                const f32x4v acc = acc2[tt][0] + acc2[tt][1];
#pragma unroll
                for (int v = 0; v < 4; ++v) pend[tt][v] = acc[v] * hsn2[tt];
            }
            pbad = 0;
#pragma unroll
            for (int v = 0; v < 4; ++v) pbad |= (rowbad[4 * g + v] ? 1u : 0u) << v;
            pm0 = m0;
            continue;
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            const f32x4v acc = acc2[tt][0] + acc2[tt][1];
            const int t = t0 + 16 * tt + c;
            const float hv = TT == 1 ? hsn : hsn2[tt];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + 4 * g + v;
                if (m < M && t < N)
                    logits[(size_t)m * N + t] = rowbad[4 * g + v] ? __builtin_nanf("") : acc[v] * hv;
            }
        }
    }
    if (DMA) store_pending();
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
    // from 4 rows on (and K up to 1024, whose codes fit a wave's registers)
    // the matrix cores; below, or for longer rows, the fp32 kernel
    const int64_t KP = (K + 63) / 64 * 64;
    if (M < 4 || KP > 1024) return launch_head_fp32(x, M, K, Qt, ldt, hs, N, logits, stream);
    const size_t shm_planes = (size_t)3 * 16 * (KP + 8) * 2;
    // waves per workgroup and token tiles per wave (each tile's activation
    // parts are built once per workgroup, each LDS read of them feeds TT
    // token tiles).  58 x 768 x 50257: one tile, 8 waves 55.4 us; two tiles,
    // 4 waves 41.4 us, 8 waves 37.9 us (130 rows: 105 -> 63 us).  The reads
    // of the activation parts from LDS were the bound.
    static const int env_tt = (int)(getenv("W4_HEAD_TT") ? atoi(getenv("W4_HEAD_TT")) : 2);
    static const int env_wv = (int)(getenv("W4_HEAD_WAVES") ? atoi(getenv("W4_HEAD_WAVES")) : 8);
    // two tiles hold the widened codes of at most 24 steps (K <= 768) in
    // registers; four tiles (bytes widened per step, one wave per SIMD) took
    // 50.1 us
    const int TTv = (env_tt == 1 || KP > 768) ? 1 : 2;
    // two tiles: the raw activation tile after the part planes
    const size_t shm = shm_planes + (TTv == 2 ? (size_t)16 * K * sizeof(float) : 0);
    const int WVv = env_wv == 8 ? 8 : 4;
    const int tokens = 16 * TTv * WVv;
    const dim3 grid((unsigned)((N + tokens - 1) / tokens));
    const int S = (int)(KP / 32);  // MFMA steps per lane group
    // more than 64 KB of dynamic LDS (K above 640) is allowed once per kernel
#define W4_HR(SV, WV, TTV)                                                                        \
    do {                                                                                          \
        static const hipError_t attr = hipFuncSetAttribute(                                      \
            reinterpret_cast<const void *>(&k_head_rows_x3<SV, WV, TTV>),                        \
            hipFuncAttributeMaxDynamicSharedMemorySize,                                          \
            3 * 16 * (32 * SV + 8) * 2 + (TTV == 2 ? 16 * 32 * SV * 4 : 0));                     \
        if (attr != hipSuccess) return attr;                                                      \
        hipLaunchKernelGGL((k_head_rows_x3<SV, WV, TTV>), grid, dim3(64 * WV), shm, stream, x,    \
                           (int)M, (int)K, Qt, (int)ldt, hs, (int)N, logits);                     \
    } while (0)
#define W4_HR_S(WV, TTV)                                                                          \
    do {                                                                                          \
        if (S <= 8) W4_HR(8, WV, TTV);                                                            \
        else if (S <= 16) W4_HR(16, WV, TTV);                                                     \
        else if (S <= 24) W4_HR(24, WV, TTV);                                                     \
        else W4_HR(32, WV, TTV);                                                                  \
    } while (0)
    if (TTv == 1 && WVv == 8) W4_HR_S(8, 1);
    else if (TTv == 1) W4_HR_S(4, 1);
    else if (WVv == 8) {
        if (S <= 8) W4_HR(8, 8, 2);
        else if (S <= 16) W4_HR(16, 8, 2);
        else W4_HR(24, 8, 2);
    } else {
        if (S <= 8) W4_HR(8, 4, 2);
        else if (S <= 16) W4_HR(16, 4, 2);
        else W4_HR(24, 4, 2);
    }
#undef W4_HR_S
#undef W4_HR
    return hipGetLastError();
}

}  // namespace w4
