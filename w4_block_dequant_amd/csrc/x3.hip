// Y = X . W_hat + bias for M >= 3 rows on the K-major layout, on the bf16
// matrix cores with fp32 accuracy (page "ONNX export, quantization and the
// browser runtime", section "Quantization", steps 1-2, and the runtime
// paragraph after them: W_hat = (q - z) * scale, fp32 matmul).
//
// Exact operands.  Within one 32-row block a column's weights are
// (q - z) * s with a single scale s, so
//   sum_{k in block} x_k * (q_k - z) * s = s * sum_{k in block} x_k * (q_k - z).
// (q - z) is an integer in [-15, 15]: exact in bf16.  Any fp32 x is exactly
// the sum of three bf16 values x = h + m + l (h = bf16(x), m = bf16(x - h),
// l = x - h - m; each difference is exact in fp32).  So the block sum is
// three v_mfma_f32_16x16x32_bf16 with exact products and fp32 accumulation,
// and the scale is applied once per block and column in fp32.  Compared with
// sum_k x_k * fl32((q_k - z) s) this only moves roundings of relative size
// 2^-24, well inside the result bound.
//
// Encoding.  The codes are turned into bf16 through the exact fp16-subnormal
// form used by the GEMV: (q - z) * 2^-24 for even k and (q - z) * 2^-20 for odd
// k (no shift for the odd nibbles); the activations of odd k are scaled by
// 2^-4 before they are split, so every product is x_k (q_k - z) 2^-24 and the
// block sum is rescaled by s * 2^24.
//
// Work split.  Lane (g, c) = (lane / 16, lane % 16).  A wave owns NT tiles of
// 16 columns; lane c of tile t is column n0 + 16 t + c and lane group g holds
// block rows 8 g .. 8 g + 7, i.e. one 32-bit word of that column's codes (each
// lane loads a whole block, 16 bytes, and a 4 x 4 transpose in LDS hands
// the words out, so a load instruction reads 64 contiguous bytes per column).  The
// four waves of a workgroup own adjacent columns and the same K range, so the
// activations' bf16 parts (the A operands, MT tiles of 16 rows) are built once
// per quad of 4 blocks in LDS and shared (one barrier per quad).  A workgroup takes QPW quads (4 blocks each)
// in straight-line code, with the loads of quad j + DQ issued before quad j is
// processed.  Workgroups along K (split-K) write partial sums that the
// fixed-order reduce kernel adds (splitk.h), so results are deterministic.
#include "common.h"
#include "epilogue.h"
#include "launch.h"
#include "splitk.h"

namespace w4 {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{a, b}, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) {
    return __builtin_bit_cast(float, v & 0xFFFF0000u);
}

template <int MT, int NT>
struct QuadLoads {
    u32x4_t w[NT];      // codes of block 4 q + g (lane group g): all 32 rows
    f32x4_t s[NT];      // the quad's four block scales
    uint32_t z[NT];     // four zero-point nibbles (16 bits)
    float2 xv[MT][4];   // this thread's activation pair, per m-tile and block
};

template <int MT, int NT, int QPW, int DQ, bool H>
__global__ __launch_bounds__(256) void k_mm_x3(const float *__restrict__ x, int M, int K,
                                               const uint8_t *__restrict__ Pq,
                                               const void *__restrict__ Ps,
                                               const uint8_t *__restrict__ Pz, int N,
                                               const float *__restrict__ bias,
                                               const float *residual, int act,
                                               float *y, int npad,
                                               float *__restrict__ part) {
    // A operands of a quad: [buffer][block][m-tile][part][lane]; two buffers
    // (one barrier per quad) while they fit, else one (two barriers per quad)
    constexpr int NBUF = MT <= 2 ? 2 : 1;
    __shared__ u32x4_t img[NBUF][4][MT * 3 * 64];
    __shared__ u32x4_t tq[4][NT * 64];       // per wave: codes of a quad, for the transpose

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int NB = K / kBlock, NQ = K / (4 * kBlock), hk = K / 2;
    const int split = blockIdx.y, splits = gridDim.y;
    const int m0 = blockIdx.z * (16 * MT);  // this workgroup's group of 16 MT rows
    const int q_begin = split * QPW;
    const int nq = min(QPW, NQ - q_begin);  // quads of this workgroup (the last may have fewer)
    const int nw = blockIdx.x * (64 * NT) + wave * (16 * NT);

    uint32_t oq[NT], os[NT], oz[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int nl = min(nw + 16 * t + c, N - 1);  // past N: re-read the last column
        oq[t] = (uint32_t)nl * (uint32_t)hk + 16u * g;
        os[t] = (uint32_t)nl * (uint32_t)NB;
        oz[t] = (uint32_t)nl * (uint32_t)(NB / 2);
    }
    // A builder role: thread = (row tid / 16 of each m-tile, k pair tid % 16).
    // Offsets are taken from this row group's first row, so they stay below
    // 64 K elements (the host keeps K below 2^22) whatever M is.
    const float *xg = x + (size_t)m0 * K;
    const int brow = tid >> 4, kp = tid & 15;
    uint32_t ox[MT];
    bool rok[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = m0 + 16 * i + brow;
        rok[i] = m < M;
        ox[i] = (uint32_t)(min(m, M - 1) - m0) * (uint32_t)K + 2u * kp;
    }
    const int slot = 16 * (kp >> 2) + brow;  // A lane holding this pair
    const int dw = kp & 3;                   // dword within that lane's 16 bytes

    auto issue = [&](int j, QuadLoads<MT, NT> &R) {
        const uint32_t q = (uint32_t)(q_begin + min(j, nq - 1));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            // offsets summed in 32 bits first: one unsigned offset from a uniform
            // base lets each load take the scalar-base form (no 64-bit address math)
            R.w[t] = load_stream<u32x4_t>(Pq + (oq[t] + 64u * q));  // block 4 q + g
            if (H) {  // four binary16 scales
                const u32x2_t h =
                    load_stream<u32x2_t>(static_cast<const char *>(Ps) + 2u * (os[t] + 4u * q));
                R.s[t] = f32x4_t{f16_bits_to_f32((uint16_t)h.x), f16_bits_to_f32((uint16_t)(h.x >> 16)),
                                 f16_bits_to_f32((uint16_t)h.y), f16_bits_to_f32((uint16_t)(h.y >> 16))};
            } else {
                R.s[t] = load_stream<f32x4_t>(static_cast<const char *>(Ps) + 4u * (os[t] + 4u * q));
            }
            R.z[t] = load_stream<uint16_t>(Pz + (oz[t] + 2u * q));
        }
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                R.xv[i][b] = *reinterpret_cast<const float2 *>(
                    reinterpret_cast<const char *>(xg) + 4u * (ox[i] + 32u * (4u * q + b)));
    };

    f32x4v acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = f32x4v{0.f, 0.f, 0.f, 0.f};
    const f32x4v zero4 = {0.f, 0.f, 0.f, 0.f};

    // straight-line over the workgroup's quads, loads DQ quads ahead
    QuadLoads<MT, NT> L[QPW];
#pragma unroll
    for (int j = 0; j < DQ && j < QPW; ++j) issue(j, L[j]);
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
        // keep each quad's loads where they are issued: DQ quads ahead, not all at once
        __builtin_amdgcn_sched_barrier(0);
        if (j + DQ < QPW) issue(j + DQ, L[j + DQ]);
        __builtin_amdgcn_sched_barrier(0);
        QuadLoads<MT, NT> &R = L[j];
        const bool live = j < nq;
        // 4 x 4 word transpose through this wave's LDS: lane (g, c) loaded all
        // of block 4 q + g; for block blk it needs word g of block 4 q + blk,
        // which lane (blk, c) holds.  Wave-private, so no barrier.
        uint32_t wq[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            tq[wave][t * 64 + lane] = R.w[t];
            const uint32_t *tw = reinterpret_cast<const uint32_t *>(tq[wave] + t * 64);
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) wq[t][blk] = tw[(blk * 16 + c) * 4 + g];
        }
        // A operands of the quad's four blocks: x split into three bf16 parts
        u32x4_t(*quad_img)[MT * 3 * 64] = img[j % NBUF];
        if (NBUF == 1 && j > 0) __syncthreads();  // previous quad's reads are done
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            uint32_t *im = reinterpret_cast<uint32_t *>(quad_img[blk]);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const bool on = live && rok[i];
                const float a0 = on ? R.xv[i][blk].x : 0.0f;
                const float a1 = on ? R.xv[i][blk].y * 0.0625f : 0.0f;  // odd k
                const uint32_t h = pack_bf16(a0, a1);
                const float r0 = a0 - bf16_lo(h), r1 = a1 - bf16_hi(h);
                const uint32_t m = pack_bf16(r0, r1);
                const uint32_t l = pack_bf16(r0 - bf16_lo(m), r1 - bf16_hi(m));
                uint32_t *base = im + ((i * 3) * 64 + slot) * 4 + dw;
                base[0] = h;
                base[64 * 4] = m;
                base[2 * 64 * 4] = l;
            }
        }
        __syncthreads();
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            // B operands: (q - z) of rows 8 g .. 8 g + 7, one per column tile
            bf16x8_t b[NT];
            float sc[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint32_t w = wq[t][blk];
                const uint32_t z = (R.z[t] >> (4 * blk)) & 15u;
                const half2_t zE = as_half2(z * 0x00010001u);
                const half2_t zO = as_half2((z << 4) * 0x00010001u);
                const uint32_t hv = w >> 8;
                const half2_t e0 = as_half2(w & 0x000F000Fu) - zE;   // k 0, 4
                const half2_t o0 = as_half2(w & 0x00F000F0u) - zO;   // k 1, 5
                const half2_t e1 = as_half2(hv & 0x000F000Fu) - zE;  // k 2, 6
                const half2_t o1 = as_half2(hv & 0x00F000F0u) - zO;  // k 3, 7
                const u32x4_t bw = {pack_bf16((float)e0.x, (float)o0.x),
                                    pack_bf16((float)e1.x, (float)o1.x),
                                    pack_bf16((float)e0.y, (float)o0.y),
                                    pack_bf16((float)e1.y, (float)o1.y)};
                b[t] = __builtin_bit_cast(bf16x8_t, bw);
                sc[t] = R.s[t][blk];  // the sums are in units of 2^-24 until the end
            }
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const u32x4_t *ai = quad_img[blk] + (i * 3) * 64 + lane;
                const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, ai[0]);
                const bf16x8_t am = __builtin_bit_cast(bf16x8_t, ai[64]);
                const bf16x8_t al = __builtin_bit_cast(bf16x8_t, ai[128]);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    f32x4v d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b[t], zero4, 0, 0, 0);
                    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, b[t], d, 0, 0, 0);
                    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b[t], d, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[i][t][v] = __builtin_fmaf(sc[t], d[v], acc[i][t][v]);
                }
            }
        }
        // Scale-accumulate here, once per quad: the accumulators are only read
        // by the guarded stores at the end, and the compiler would otherwise
        // sink every block's FMAs there, keeping all MFMA results live.  An
        // empty asm that reads and writes each accumulator pins them in place;
        // within the quad the four blocks' MFMA chains are free to overlap.
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v) asm volatile("" : "+v"(acc[i][t][v]));
    }

    // lane (g, c) holds D[4 g + v][c] of each (m-tile, column tile), in units
    // of 2^-24 (the code encoding): the exact power-of-two rescale comes off
    // here, after the block scales, so a large scale cannot overflow early.
    // No lane leaves before the SwiGLU exchange: column pair (c, c + 1), c
    // even, is lanes (l, l + 1) of the same row group.
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int n = nw + 16 * t + c;
            const float bn = (splits == 1 && bias && n < N) ? bias[n] : 0.0f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + 16 * i + 4 * g + v;
                const bool in = n < N && m < M;
                const float r = acc[i][t][v] * 16777216.0f;
                if (splits > 1) {
                    if (in) part[((size_t)split * M + m) * npad + n] = r;
                } else if (act == W4_ACT_SWIGLU) {
                    const float tv = r + bn;
                    const float up = __shfl_down(tv, 1);
                    if (in && (c & 1) == 0)
                        ep_store_glu(tv, up, residual, y, (size_t)m * (N / 2) + n / 2);
                } else if (in) {
                    ep_store(r + bn, act, residual, y, (size_t)m * N + n);
                }
            }
        }
}

// Whole-K variant for 3 <= M <= 16 rows: one launch per matmul, no partial
// sums in memory.  A workgroup owns 16 TPW columns and all of K; its W waves
// take the quads (4 blocks) q = wave, wave + W, ... and their 16 x 16 tiles
// are added in LDS in wave order at the end (deterministic).  Per quad a
// wave converts the codes (the 4 x 4 word transpose of k_mm_x3) and builds
// the bf16 parts of the activations of its own quad in a wave-private LDS
// image, so the workgroup splits each activation once and needs no barrier
// inside the K loop.
//
// Only the first MB >= M rows of the A operand are built (MB = 4, 8 or 16);
// A lanes of rows MB .. 15 read row MB - 1 again, and every row >= M is
// dropped at the store (an MFMA row depends on that row of A only).
//
// Exact parts.  The split truncates: h = x with the low 16 bits cleared, r =
// x - h (exact: the low 16 bits of the significand), m = r truncated the
// same way, l = r - m.  h, m and l hold 8 significant bits each, so each is
// exactly a bf16 (the upper half of its fp32 pattern) and x = h + m + l.
//
// Codes.  (q - z) is formed as a normal fp16: a nibble in bits 0-3 of a half
// ORed into 0x6400 (1024) reads as 1024 + q, a nibble in bits 4-7 ORed into
// 0x5400 (64, mantissa unit 1/16) reads as 64 + q; subtracting 1024 + z or
// 64 + z in packed fp16 leaves q - z exactly, which widens to fp32 and
// narrows to bf16 exactly.  So no power of two is carried and each block sum
// is scaled by s alone.
template <int TPW, int NBLD>
struct KQuadLoads {
    u32x4_t w[TPW];        // codes of block 4 q + g (lane group g), per column tile
    f32x4_t s[TPW];        // the quad's four block scales
    uint32_t z[TPW];       // four zero-point nibbles (16 bits)
    f32x4_t xa[NBLD][2];   // 8 activations per A image this lane builds
};

// (a & m) | o in one instruction.  VOP3 takes no literal on gfx950, so the
// compiler would emit an AND and an OR with two literals; with m and o held
// in registers (loop invariants) it is one v_and_or_b32.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
    uint32_t d;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(m), "v"(o));
    return d;
}

// c + (fp16 half of h) in fp32 with one rounding (v_fma_mix_f32, the half
// widened exactly).  With h = 1024 + q or 64 + q (exact fp16 integers) and
// c = -(1024 + z) or -(64 + z), the result is q - z exactly.
__device__ __forceinline__ float mix_lo(uint32_t h, float c) {
    float d;
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(c));
    return d;
}
__device__ __forceinline__ float mix_hi(uint32_t h, float c) {
    float d;
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(c));
    return d;
}

__device__ __forceinline__ uint32_t hi16_pair(float lo, float hi) {
    // (upper half of lo) | (upper half of hi) << 16: two truncated bf16
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi),
                                 __builtin_bit_cast(uint32_t, lo), 0x07060302u);
}
__device__ __forceinline__ float trunc_rest(float v) {
    // v minus v truncated to bf16 (exact)
    return v - __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) & 0xFFFF0000u);
}

template <int MB, int TPW, int W, int D, bool H, bool P3, int NQC>
__global__ __launch_bounds__(64 * W) void k_mm_x3k(const float *__restrict__ x, int M, int K,
                                                   const uint8_t *__restrict__ Pq,
                                                   const void *__restrict__ Ps,
                                                   const uint8_t *__restrict__ Pz, int N,
                                                   const float *__restrict__ bias,
                                                   const float *residual, int act, float *y) {
    // row group blockIdx.y: rows m0 .. m0 + MB - 1 (M > MB only with MB = 16)
    {
        const int m0 = blockIdx.y * MB;
        const int nout = act == W4_ACT_SWIGLU ? N / 2 : N;
        M = min(M - m0, MB);
        x += (size_t)m0 * K;
        y += (size_t)m0 * nout;
        if (residual) residual += (size_t)m0 * nout;
    }
    constexpr int ABLK = 16 / MB;  // blocks per A image: MB rows x ABLK blocks = 64 lanes x 8
    constexpr int NBLD = 4 / ABLK;  // A images per quad
    constexpr int TQ_BYTES = TPW * 64 * 16;
    constexpr int PART_BYTES = ABLK * MB * 64;
    // part planes 16 bytes apart in the bank order under P3, where one read
    // instruction takes rows of two planes at once (no two-way bank conflict)
    constexpr int PSTRIDE = PART_BYTES + (P3 ? 16 : 0);
    constexpr int WAVE_BYTES = TQ_BYTES + 3 * PSTRIDE;
    static_assert(WAVE_BYTES >= TPW * 64 * 16, "the wave partials fit the wave's area");
    __shared__ __attribute__((aligned(16))) unsigned char lds[W * WAVE_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int NB = K / kBlock, NQ = K / (4 * kBlock), hk = K / 2;
    const int n0 = blockIdx.x * (16 * TPW);
    u32x4_t *tq = reinterpret_cast<u32x4_t *>(lds + wave * WAVE_BYTES);
    unsigned char *img = lds + wave * WAVE_BYTES + TQ_BYTES;

    uint32_t oq[TPW], os[TPW], oz[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int nl = min(n0 + 16 * t + c, N - 1);  // past N: re-read the last column
        oq[t] = (uint32_t)nl * (uint32_t)hk + 16u * g;
        os[t] = (uint32_t)nl * (uint32_t)NB;
        oz[t] = (uint32_t)nl * (uint32_t)(NB / 2);
    }
    // A builder: lane = (image block bb, row bm, slot group bg), 8 activations;
    // lane l writes bytes 16 l .. 16 l + 15 of each part plane, so a write
    // instruction covers consecutive LDS banks (no bank conflict)
    const int bb = lane / (4 * MB), bm = (lane >> 2) % MB, bg = lane & 3;
    const uint32_t ox = (uint32_t)min(bm, M - 1) * (uint32_t)K + 32u * bb + 8u * bg;
    uint32_t *const wimg = reinterpret_cast<uint32_t *>(img + (bb * MB + bm) * 64 + bg * 16);
    // A reader: lane (g, c) takes row min(c, MB - 1), slots 8 g .. 8 g + 7
    // P3 (at most 4 rows): A row c is part c / 4 (h, m, l) of row c % 4, so
    // one MFMA per block forms all three part sums (rows 12-15 repeat the l
    // part and are never read); lane group p then holds part p's sums.
    static_assert(!P3 || MB == 4, "three parts share one MFMA only for 4 rows");
    const int aoff = P3 ? min(c >> 2, 2) * PSTRIDE + (c & 3) * 64 + g * 16
                        : min(c, MB - 1) * 64 + g * 16;

    const int nq = wave < NQ ? (NQ - 1 - wave) / W + 1 : 0;  // this wave's quads
    // masks and fp16 bases of the code conversion, in registers
    uint32_t kLoMask = 0x000F000Fu, kHiMask = 0x00F000F0u, kLoBase = 0x64006400u,
             kHiBase = 0x54005400u;
    asm volatile("" : "+v"(kLoMask), "+v"(kHiMask), "+v"(kLoBase), "+v"(kHiBase));

    auto issue = [&](int i, KQuadLoads<TPW, NBLD> &R) {
        const uint32_t q = (uint32_t)(wave + W * min(i, nq - 1));
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            R.w[t] = load_stream<u32x4_t>(Pq + (oq[t] + 64u * q));
            if (H) {
                const u32x2_t h =
                    load_stream<u32x2_t>(static_cast<const char *>(Ps) + 2u * (os[t] + 4u * q));
                R.s[t] = f32x4_t{f16_bits_to_f32((uint16_t)h.x), f16_bits_to_f32((uint16_t)(h.x >> 16)),
                                 f16_bits_to_f32((uint16_t)h.y), f16_bits_to_f32((uint16_t)(h.y >> 16))};
            } else {
                R.s[t] = load_stream<f32x4_t>(static_cast<const char *>(Ps) + 4u * (os[t] + 4u * q));
            }
            R.z[t] = load_stream<uint16_t>(Pz + (oz[t] + 2u * q));
        }
#pragma unroll
        for (int b = 0; b < NBLD; ++b) {
            const char *xp = reinterpret_cast<const char *>(x) +
                             4u * (ox + 128u * q + 32u * ABLK * b);
            R.xa[b][0] = *reinterpret_cast<const f32x4_t *>(xp);
            R.xa[b][1] = *reinterpret_cast<const f32x4_t *>(xp + 16);
        }
    };

    f32x4v acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = f32x4v{0.f, 0.f, 0.f, 0.f};
    const f32x4v zero4 = {0.f, 0.f, 0.f, 0.f};

    // one quad's arithmetic on loads already issued into R
    auto process = [&](KQuadLoads<TPW, NBLD> &R) {
        // codes: lane (g, c) holds block 4 q + g of its column; word g
        // of block 4 q + blk is with lane (blk, c)
        uint32_t wq[TPW][4];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            tq[t * 64 + lane] = R.w[t];
            const uint32_t *tw = reinterpret_cast<const uint32_t *>(tq + t * 64);
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) wq[t][blk] = tw[(blk * 16 + c) * 4 + g];
        }
#pragma unroll
        for (int b = 0; b < NBLD; ++b) {
            // A image b: the three bf16 parts of this lane's 8 activations
            const float *f = reinterpret_cast<const float *>(&R.xa[b][0]);
            u32x4_t ph, pm, pl;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float a0 = f[2 * p], a1 = f[2 * p + 1];
                const float r0 = trunc_rest(a0), r1 = trunc_rest(a1);
                ph[p] = hi16_pair(a0, a1);
                pm[p] = hi16_pair(r0, r1);
                pl[p] = hi16_pair(trunc_rest(r0), trunc_rest(r1));
            }
            *reinterpret_cast<u32x4_t *>(wimg) = ph;
            *reinterpret_cast<u32x4_t *>(wimg + PSTRIDE / 4) = pm;
            *reinterpret_cast<u32x4_t *>(wimg + 2 * PSTRIDE / 4) = pl;
#pragma unroll
            for (int ib = 0; ib < ABLK; ++ib) {
                const int blk = b * ABLK + ib;
                const unsigned char *ap = img + ib * MB * 64 + aoff;
                const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(ap));
                bf16x8_t am, al;
                if (!P3) {
                    am = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(ap + PSTRIDE));
                    al = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(ap + 2 * PSTRIDE));
                }
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    const uint32_t w = wq[t][blk];
                    // -(1024 + z) and -(64 + z) as fp32 bit patterns (z
                    // lands in the mantissa bits of unit 1)
                    const uint32_t z = (R.z[t] >> (4 * blk)) & 15u;
                    const float cE = __builtin_bit_cast(float, 0xC4800000u | (z << 13));
                    const float cO = __builtin_bit_cast(float, 0xC2800000u | (z << 17));
                    const uint32_t hv = w >> 8;
                    const uint32_t e0 = and_or(w, kLoMask, kLoBase);   // 1024 + q, k 0 and 4
                    const uint32_t o0 = and_or(w, kHiMask, kHiBase);   // 64 + q, k 1 and 5
                    const uint32_t e1 = and_or(hv, kLoMask, kLoBase);  // k 2 and 6
                    const uint32_t o1 = and_or(hv, kHiMask, kHiBase);  // k 3 and 7
                    // q - z is a small integer: its fp32 pattern's upper
                    // half is its bf16 pattern (pairs packed by v_perm)
                    const u32x4_t bw = {hi16_pair(mix_lo(e0, cE), mix_lo(o0, cO)),
                                        hi16_pair(mix_lo(e1, cE), mix_lo(o1, cO)),
                                        hi16_pair(mix_hi(e0, cE), mix_hi(o0, cO)),
                                        hi16_pair(mix_hi(e1, cE), mix_hi(o1, cO))};
                    const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, bw);
                    f32x4v dd;
                    if (P3) {
                        dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv, zero4, 0, 0, 0);
                    } else {
                        dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bv, zero4, 0, 0, 0);
                        dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, bv, dd, 0, 0, 0);
                        dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv, dd, 0, 0, 0);
                    }
                    const float sc = R.s[t][blk];
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[t][v] = __builtin_fmaf(sc, dd[v], acc[t][v]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) asm volatile("" : "+v"(acc[t][v]));
    };

    if (nq > 0) {
        if constexpr (NQC > 0) {
            // Every wave has exactly NQC quads (the plan checks it), so the
            // loop unrolls into straight-line code: D quads in flight, each
            // wait covers only the oldest quad's loads (a loop with the
            // loads under a runtime condition gets a full wait at its head).
            KQuadLoads<TPW, NBLD> L[D];
#pragma unroll
            for (int d = 0; d < D; ++d) issue(d, L[d]);
#pragma unroll
            for (int i = 0; i < NQC; ++i) {
                process(L[i % D]);
                if (i + D < NQC) issue(i + D, L[i % D]);
            }
        } else {
            KQuadLoads<TPW, NBLD> L[D];
#pragma unroll
            for (int d = 0; d < D; ++d) issue(d, L[d]);
            for (int i0 = 0; i0 < nq; i0 += D) {
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    if (i0 + d >= nq) break;
                    process(L[d]);
                    if (i0 + d + D < nq) issue(i0 + d + D, L[d]);
                }
            }
        }
    }

    // Wave partials through LDS (over the waves' areas, once every wave is
    // done with them), added in wave order.  Lane (g, c) of tile t holds
    // rows 4 g .. 4 g + 3 of column 16 t + c.
    __syncthreads();
    f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);
#pragma unroll
    for (int t = 0; t < TPW; ++t) red[(wave * TPW + t) * 64 + lane] = f32x4_t{acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
    __syncthreads();
    const float *rf = reinterpret_cast<const float *>(lds);
    auto total = [&](int m, int nl) {
        float v = 0.0f;
        if (P3) {  // m < 4: the h, m and l sums sit in lane groups 0, 1, 2
            const int idx = ((nl >> 4) * 64 + (nl & 15)) * 4 + m;
#pragma unroll
            for (int w2 = 0; w2 < W; ++w2) {
                const float *r = rf + w2 * TPW * 256 + idx;
                v += r[0] + r[64] + r[128];
            }
        } else {
            const int idx = ((nl >> 4) * 64 + (m >> 2) * 16 + (nl & 15)) * 4 + (m & 3);
#pragma unroll
            for (int w2 = 0; w2 < W; ++w2) v += rf[w2 * TPW * 256 + idx];
        }
        return v;
    };
    constexpr int CW = 16 * TPW;
    if (act == W4_ACT_SWIGLU) {
        for (int o = tid; o < M * (CW / 2); o += 64 * W) {
            const int m = o / (CW / 2), nl = 2 * (o % (CW / 2)), n = n0 + nl;
            if (n >= N) continue;
            const float gate = total(m, nl) + (bias ? bias[n] : 0.0f);
            const float up = total(m, nl + 1) + (bias ? bias[n + 1] : 0.0f);
            ep_store_glu(gate, up, residual, y, (size_t)m * (N / 2) + n / 2);
        }
    } else {
        for (int o = tid; o < M * CW; o += 64 * W) {
            const int m = o / CW, nl = o % CW, n = n0 + nl;
            if (n >= N) continue;
            ep_store(total(m, nl) + (bias ? bias[n] : 0.0f), act, residual, y, (size_t)m * N + n);
        }
    }
}

}  // namespace

template <int MB, int TPW, int W, int D, bool H, int NQC>
void launch_x3k_n(bool p3, dim3 grid, hipStream_t stream, const float *x, int64_t M, int64_t K,
                  const uint8_t *Pq, const void *Ps, const uint8_t *Pz, int64_t N,
                  const float *bias, const float *residual, int act, float *y) {
    if constexpr (MB == 4) {
        if (p3) {
            hipLaunchKernelGGL((k_mm_x3k<MB, TPW, W, D, H, true, NQC>), grid, dim3(64 * W), 0, stream,
                               x, (int)M, (int)K, Pq, Ps, Pz, (int)N, bias, residual, act, y);
            return;
        }
    }
    hipLaunchKernelGGL((k_mm_x3k<MB, TPW, W, D, H, false, NQC>), grid, dim3(64 * W), 0, stream, x,
                       (int)M, (int)K, Pq, Ps, Pz, (int)N, bias, residual, act, y);
}

template <int MB, int TPW, int W, int D, bool H>
void launch_x3k(bool p3, int nqc, dim3 grid, hipStream_t stream, const float *x, int64_t M,
                int64_t K, const uint8_t *Pq, const void *Ps, const uint8_t *Pz, int64_t N,
                const float *bias, const float *residual, int act, float *y) {
    // straight-line variants for 3 and 8 quads per wave (K = 3072 and 8192
    // with 8 waves), fp32 scales
    if constexpr (!H && W == 8 && D <= 3) {
        if (nqc == 3) {
            launch_x3k_n<MB, TPW, W, D, H, 3>(p3, grid, stream, x, M, K, Pq, Ps, Pz, N, bias,
                                              residual, act, y);
            return;
        }
        if (nqc == 8) {
            launch_x3k_n<MB, TPW, W, D, H, 8>(p3, grid, stream, x, M, K, Pq, Ps, Pz, N, bias,
                                              residual, act, y);
            return;
        }
    }
    launch_x3k_n<MB, TPW, W, D, H, 0>(p3, grid, stream, x, M, K, Pq, Ps, Pz, N, bias, residual,
                                      act, y);
}

hipError_t launch_mm_x3(const X3Plan &p, const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                        const void *Ps, bool f16, const uint8_t *Pz, int64_t N, const float *bias,
                        const float *residual, int act, float *y, void *workspace,
                        hipStream_t stream) {
    if (p.kind == X3Plan::kFullK) {
        const dim3 grid((unsigned)p.col_wgs, (unsigned)p.mgroups);
        bool done = false;
#define W4_X3K(MBV, TPWV, WV, DV)                                                                  \
    if (!done && p.mb == MBV && p.nt == TPWV && p.waves == WV && (p.dq == DV || p.dq == 0)) {      \
        if (f16)                                                                                    \
            launch_x3k<MBV, TPWV, WV, DV, true>(p.p3, p.nqc, grid, stream, x, M, K, Pq, Ps, Pz, N, bias,    \
                                                residual, act, y);                                  \
        else                                                                                        \
            launch_x3k<MBV, TPWV, WV, DV, false>(p.p3, p.nqc, grid, stream, x, M, K, Pq, Ps, Pz, N, bias,   \
                                                 residual, act, y);                                 \
        done = true;                                                                                \
    }
#define W4_X3K_W(MBV, TPWV, DV) W4_X3K(MBV, TPWV, 4, DV) W4_X3K(MBV, TPWV, 8, DV)
#define W4_X3K_W3(MBV, DV) W4_X3K(MBV, 1, 4, DV) W4_X3K(MBV, 1, 8, DV) W4_X3K(MBV, 1, 16, DV)
        // the first instantiation of a row count is its default depth
        W4_X3K_W3(4, 1) W4_X3K_W3(4, 2) W4_X3K_W3(4, 4) W4_X3K(4, 1, 8, 3) W4_X3K_W(4, 2, 1)
        W4_X3K_W(4, 2, 3)
        W4_X3K_W3(8, 1) W4_X3K_W3(8, 2) W4_X3K_W(8, 2, 1) W4_X3K_W(8, 2, 2)
        W4_X3K_W3(16, 1) W4_X3K_W3(16, 2) W4_X3K_W(16, 2, 1) W4_X3K_W(16, 2, 2)
#undef W4_X3K_W3
#undef W4_X3K_W
#undef W4_X3K
        if (!done) return hipErrorInvalidValue;
        return hipGetLastError();
    }
    const dim3 grid((unsigned)p.col_wgs, (unsigned)p.splits, (unsigned)p.mgroups);
    float *part = p.splits > 1 ? static_cast<float *>(workspace) : nullptr;
    bool launched = false;
#define W4_X3(MTV, NTV, QV, DQV)                                                                \
    if (!launched && p.mt == MTV && p.nt == NTV && p.quads_per_wg == QV && p.dq == DQV) {       \
        if (f16)                                                                                \
            hipLaunchKernelGGL((k_mm_x3<MTV, NTV, QV, DQV, true>), grid, dim3(256), 0, stream, x, \
                               (int)M, (int)K, Pq, Ps, Pz, (int)N, bias, residual, act, y,       \
                               (int)p.npad, part);                                              \
        else                                                                                    \
            hipLaunchKernelGGL((k_mm_x3<MTV, NTV, QV, DQV, false>), grid, dim3(256), 0, stream,   \
                               x, (int)M, (int)K, Pq, Ps, Pz, (int)N, bias, residual, act, y,    \
                               (int)p.npad, part);                                              \
        launched = true;                                                                        \
    }
#define W4_X3_Q(MTV, NTV, DQV)                                                                  \
    W4_X3(MTV, NTV, 1, DQV) W4_X3(MTV, NTV, 2, DQV) W4_X3(MTV, NTV, 3, DQV)                     \
    W4_X3(MTV, NTV, 4, DQV) W4_X3(MTV, NTV, 6, DQV) W4_X3(MTV, NTV, 8, DQV)                     \
    W4_X3(MTV, NTV, 12, DQV)
    W4_X3_Q(1, 1, 2) W4_X3_Q(2, 1, 3) W4_X3_Q(3, 1, 2) W4_X3_Q(4, 1, 2)
    W4_X3_Q(1, 2, 3) W4_X3_Q(2, 2, 2) W4_X3_Q(1, 1, 1) W4_X3_Q(1, 1, 3)
#undef W4_X3_Q
#undef W4_X3
    if (!launched) return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_reduce(part, p.splits, M, N, p.npad, bias, nullptr, 1.0f, y, stream,
                                residual, act);
}

}  // namespace w4
