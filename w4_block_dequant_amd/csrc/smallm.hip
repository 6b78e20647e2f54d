// M > 1 (prefill rows, batched decode): dequantize to LDS, then fp32 MFMA.
//
// The method (page "ONNX export, quantization and the browser runtime",
// section "Quantization", steps 1-2, and the runtime paragraph after them)
// computes Y = X . W_hat + bias in fp32 with W_hat = (q - z) * scale.  With
// M >= 16 rows the product is a dense contraction, so it runs on
// v_mfma_f32_16x16x4_f32 (true fp32: no reduced-precision inputs).
//
// A workgroup (4 waves) owns a 256-column tile and a range of K-blocks.  Per
// 32-row block every thread loads 4 rows x 8 columns of packed codes (rows of
// 128 contiguous bytes across 32 threads), dequantizes them exactly --
// (q - z) as an fp16-subnormal pair, widened to the exact integer, times the
// scale: fl32((q - z) * scale), the same value the oracle forms -- and stores
// the fp32 tile in one of two LDS buffers.  After one barrier each wave runs
// its 64 columns (4 MFMA n-tiles) against up to 4 MFMA m-tiles of X, reading
// its B operands with ds_read_b128, while the next block's loads are in
// flight.  Workgroups along K write partial sums that a second kernel adds
// in split order (splitk.h).
#include "common.h"
#include "launch.h"
#include "splitk.h"

namespace w4 {

hipError_t launch_matmul_generic(const float *x, int64_t M, int64_t K, const uint8_t *Wq,
                                 const float *scales, const uint8_t *zeros, int64_t N,
                                 const float *bias, float *y, hipStream_t stream);

namespace {

constexpr int kTN = 256;     // columns per workgroup tile
constexpr int kRowsPad = 256;  // LDS row stride (floats)

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Operand layout of v_mfma_f32_16x16x4_f32 (one 16x16 block):
//   A (16 x 4): lane l holds A[l % 16][l / 16]
//   B (4 x 16): lane l holds B[l / 16][l % 16]
//   D (16 x 16): lane l, register v holds D[4 * (l / 16) + v][l % 16]
// The k index of A and B only has to agree per lane group, so lane group kq
// at step t stands for block row 8 * kq + t.
//
// Pipeline: a ring of D register sets holds the raw loads (codes, scales,
// zero points and the block's x tile) of the next D blocks.  Each step
// dequantizes one set into LDS (weights as fp32, x as an MFMA-ready tile),
// refills the set with the block D steps ahead, then runs the MFMAs from LDS,
// so global latency is covered by D blocks of MFMA work.  The ring is
// unrolled, so every index is static; steps past the workgroup's last block
// re-read that block and store zero scales and zero activations, which adds
// nothing to the sums and keeps control flow uniform.
constexpr int kXPad = 36;  // LDS row stride of the x tile (floats): conflict-free b128 reads

template <int MT>
struct MmaLoads {
    uint32_t w[4];
    f32x4_t s[2];
    uint32_t z;
    float2 xv[MT];
};

template <int MT, int D>
__global__ __launch_bounds__(256) void k_mm_mfma(
    const float *__restrict__ x, int64_t M, int64_t K, const uint8_t *__restrict__ Wq,
    const float *__restrict__ scales, const uint8_t *__restrict__ zeros, int64_t N,
    const float *__restrict__ bias, float *__restrict__ y, int64_t tiles, int64_t splits,
    int64_t bpw, int64_t npad, float *__restrict__ part) {
    __shared__ float Ws[2][kBlock * kRowsPad];
    __shared__ float Xs[2][16 * MT * kXPad];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int kq = lane >> 4, c = lane & 15;
    const int64_t wg = blockIdx.x;
    const int64_t tile = wg % tiles;
    const int64_t split = (wg / tiles) % splits;
    const int64_t mg = wg / (tiles * splits);
    const int64_t n0 = tile * kTN;
    const int64_t m0 = mg * 64;
    const int64_t NB = K / kBlock;
    const int64_t b_begin = split * bpw;
    const int64_t b_end = min(b_begin + bpw, NB);
    const int64_t half = N / 2;

    // loader role: 8 columns (4 packed bytes) x 4 rows; x tile element pairs
    const int li = tid & 31, lg = tid >> 5;
    const int64_t lcol = min(n0 + 8 * li, N - 8);  // clamped: columns past N store zeros
    const bool lok = n0 + 8 * li < N;

    auto issue = [&](int64_t b, MmaLoads<MT> &R) {
        const uint8_t *wp = Wq + (b * kBlock + 4 * lg) * half + lcol / 2;
#pragma unroll
        for (int r = 0; r < 4; ++r) R.w[r] = load_stream<uint32_t>(wp + r * half);
        const float *sp = scales + b * N + lcol;
        R.s[0] = *reinterpret_cast<const f32x4_t *>(sp);
        R.s[1] = *reinterpret_cast<const f32x4_t *>(sp + 4);
        R.z = *reinterpret_cast<const uint32_t *>(zeros + b * half + lcol / 2);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int e = tid + 256 * i;            // pair index in the [16 MT][32] tile
            const int64_t row = min(m0 + e / 16, M - 1);
            R.xv[i] = *reinterpret_cast<const float2 *>(x + row * K + b * kBlock + 2 * (e % 16));
        }
    };
    auto store = [&](const MmaLoads<MT> &R, bool live, float *wbuf, float *xbuf) {
        f32x4_t o[4][2];
        const NibblePairs zp = nibble_pairs(R.z);
        const bool on = live && lok;
        float su[8];  // the scale (0 for columns past N or a dead step)
#pragma unroll
        for (int j = 0; j < 8; ++j) su[j] = on ? R.s[j >> 2][j & 3] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const NibblePairs qp = nibble_pairs(R.w[r]);
            float w[8];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // (q - z) first (exact: a small integer), then the one rounding
                // of fl32((q - z) * scale); scaling the scale by 2^24 instead
                // would overflow for scales of 2^104 and up
                const half2_t d = qp.p[m] - zp.p[m];
                w[m] = ((float)d.x * nibble_unscale(m)) * su[m];
                w[m + 4] = ((float)d.y * nibble_unscale(m + 4)) * su[m + 4];
            }
            o[r][0] = f32x4_t{w[0], w[1], w[2], w[3]};
            o[r][1] = f32x4_t{w[4], w[5], w[6], w[7]};
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float *dst = wbuf + (4 * lg + r) * kRowsPad + 8 * li;
            *reinterpret_cast<f32x4_t *>(dst) = o[r][0];
            *reinterpret_cast<f32x4_t *>(dst + 4) = o[r][1];
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int e = tid + 256 * i;
            const bool rok = live && (m0 + e / 16 < M);
            const float2 v = rok ? R.xv[i] : make_float2(0.0f, 0.0f);
            *reinterpret_cast<float2 *>(xbuf + (e / 16) * kXPad + 2 * (e % 16)) = v;
        }
    };

    f32x4v acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4v{0.f, 0.f, 0.f, 0.f};

    MmaLoads<MT> ring[D];
#pragma unroll
    for (int j = 0; j < D; ++j) issue(min(b_begin + j, b_end - 1), ring[j]);
    int buf = 0;
    for (int64_t b = b_begin; b < b_end; b += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int64_t bb = b + j;
            store(ring[j], bb < b_end, Ws[buf], Xs[buf]);
            __syncthreads();
            issue(min(bb + D, b_end - 1), ring[j]);
            const float *bs = Ws[buf] + 64 * wave + 4 * c;
            const float *xs = Xs[buf] + c * kXPad + 8 * kq;
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                f32x4_t xa[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    xa[mt] = *reinterpret_cast<const f32x4_t *>(xs + 16 * mt * kXPad + 4 * t2);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const f32x4_t bv =
                        *reinterpret_cast<const f32x4_t *>(bs + (8 * kq + 4 * t2 + t) * kRowsPad);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < 4; ++nt)
                            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[mt][t], bv[nt],
                                                                                 acc[mt][nt], 0, 0, 0);
                }
            }
            buf ^= 1;
        }
    }

    // lane holds D[4 kq + v][c] of each (mt, nt): row m0 + 16 mt + 4 kq + v,
    // column n0 + 64 wave + 4 c + nt
    const int64_t rows = min((int64_t)64, M - m0);
    float *pp = splits == 1 ? nullptr : part + split * (M * npad);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int64_t n = n0 + 64 * wave + 4 * c + nt;
            const float bn = (splits == 1 && bias && n < N) ? bias[n] : 0.0f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t mr = 16 * mt + 4 * kq + v;
                if (mr >= rows) continue;
                if (splits == 1) {
                    if (n < N) y[(m0 + mr) * N + n] = acc[mt][nt][v] + bn;
                } else {
                    pp[(m0 + mr) * npad + n] = acc[mt][nt][v];
                }
            }
        }
}

}  // namespace

hipError_t launch_small_m(const SmallMPlan &p, const float *x, int64_t M, int64_t K,
                          const uint8_t *Wq, const float *scales, const uint8_t *zeros,
                          int64_t N, const float *bias, float *y, void *workspace,
                          hipStream_t stream) {
    switch (p.kind) {
    case SmallMPlan::kEmpty:
        return hipSuccess;
    case SmallMPlan::kBiasOnly:
        return launch_bias_fill(bias, M, N, y, stream);
    case SmallMPlan::kGeneric:
        return launch_matmul_generic(x, M, K, Wq, scales, zeros, N, bias, y, stream);
    case SmallMPlan::kMfma:
        break;
    }
    float *part = p.splits > 1 ? static_cast<float *>(workspace) : nullptr;
    const dim3 grid((unsigned)(p.tiles * p.splits * p.mgroups));
#define W4_MFMA_CASE(MTV, DV)                                                                   \
    if (p.mtiles == MTV && p.depth == DV) {                                                     \
        hipLaunchKernelGGL((k_mm_mfma<MTV, DV>), grid, dim3(256), 0, stream, x, M, K, Wq, scales, \
                           zeros, N, bias, y, p.tiles, p.splits, p.blocks_per_wg, p.npad, part); \
        launched = true;                                                                        \
    }
    bool launched = false;
    W4_MFMA_CASE(1, 1) W4_MFMA_CASE(1, 2) W4_MFMA_CASE(1, 3)
    W4_MFMA_CASE(2, 1) W4_MFMA_CASE(2, 2) W4_MFMA_CASE(2, 3)
    W4_MFMA_CASE(3, 1) W4_MFMA_CASE(3, 2)
    W4_MFMA_CASE(4, 1) W4_MFMA_CASE(4, 2)
    if (!launched) return hipErrorInvalidValue;
#undef W4_MFMA_CASE
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_reduce(part, p.splits, M, N, p.npad, bias, nullptr, 1.0f, y, stream);
}

}  // namespace w4
