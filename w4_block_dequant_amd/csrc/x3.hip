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
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{a, b}, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) {
    return __builtin_bit_cast(float, v & 0xFFFF0000u);
}

// (a & m) | (b & ~m) in one instruction
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) {
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(a), "v"(b));
    return r;
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
    // A builder role: thread = (row tid / 16 of each m-tile, k pair tid % 16)
    const int brow = tid >> 4, kp = tid & 15;
    uint32_t ox[MT];
    bool rok[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = m0 + 16 * i + brow;
        rok[i] = m < M;
        ox[i] = (uint32_t)min(m, M - 1) * (uint32_t)K + 2u * kp;
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
                    reinterpret_cast<const char *>(x) + 4u * (ox[i] + 32u * (4u * q + b)));
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
                sc[t] = R.s[t][blk] * 16777216.0f;
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

    // lane (g, c) holds D[4 g + v][c] of each (m-tile, column tile).  No lane
    // leaves before the SwiGLU exchange: column pair (c, c + 1), c even, is
    // lanes (l, l + 1) of the same row group.
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
                if (splits > 1) {
                    if (in) part[((size_t)split * M + m) * npad + n] = acc[i][t][v];
                } else if (act == W4_ACT_SWIGLU) {
                    const float tv = acc[i][t][v] + bn;
                    const float up = __shfl_down(tv, 1);
                    if (in && (c & 1) == 0)
                        ep_store_glu(tv, up, residual, y, (size_t)m * (N / 2) + n / 2);
                } else if (in) {
                    ep_store(acc[i][t][v] + bn, act, residual, y, (size_t)m * N + n);
                }
            }
        }
}

// fp16 form of the same product, for a single 16-row tile (M <= 16): the
// workgroup's activations are prepared before its first quad.
//
// Codes.  (w & 0x000F000F) | 0x64006400 read as two fp16 numbers is
// (1024 + q, 1024 + q') for the nibbles at bits 0 and 16 of a word, and
// (w & 0x00F000F0) | 0x64006400 is (1024 + 16 q, ...) for those at bits 4 and
// 20.  Subtracting the zero point's pair (1024 + z or 1024 + 16 z) leaves
// q - z or 16 (q - z), exact normal fp16 numbers: one bit-field insert and
// half a packed subtraction per code, against two and a half operations per
// code for the bf16 form.  Lane group g gives its MFMA slots the 8 codes of
// word g in the order the pairs fall: k = 0 4 1 5 2 6 3 7 of the word.
//
// Activations.  Each row is multiplied by its own power of two 2^a, chosen so
// that the row's largest |x| within the workgroup's K range lies in
// [2^14, 2^15) (odd k by 2^(a-4), for the 16 (q - z) codes), and split into
// three fp16 parts h + m + l by round-to-nearest and exact fp32 differences.
// What the parts leave out is at most 2^-33 |x| + 2^-39 max|x| per
// activation, max over that row and K range; the products with the codes are
// exact in fp32 and the block sums fp32, as in the bf16 kernel, and each
// row's sums are multiplied by 2^-a at the end.  So the result is within the
// matmul bound unless a row's largest activation in a workgroup's K range
// (at most 512 values) exceeds about 5 * 10^6 times that row's |w|-weighted
// average there.  All of the workgroup's A operands are built in LDS while
// its first weights are in flight, so the quad loop has no barrier; each
// lane loads the scales and zero points of one quad for all the workgroup's
// quads, and the quad loop takes them from that lane.  NaN or infinite
// activations give NaN outputs.
template <int MT, int NT, int QPW, int DQ, bool H>
__global__ __launch_bounds__(256) void k_mm_h3(const float *__restrict__ x, int M, int K,
                                               const uint8_t *__restrict__ Pq,
                                               const void *__restrict__ Ps,
                                               const uint8_t *__restrict__ Pz, int N,
                                               const float *__restrict__ bias,
                                               const float *residual, int act,
                                               float *y, int npad,
                                               float *__restrict__ part) {
    __shared__ u32x4_t img[QPW][4][MT * 3 * 64];  // [quad][block][m-tile][part][lane]
    __shared__ u32x4_t tq[4][NT * 64];            // per wave: codes of a quad, for the transpose
    __shared__ int srow[MT][16];                  // each row's scale exponent
    static_assert(QPW <= 4, "one scale load per lane covers at most 4 quads");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int NB = K / kBlock, hk = K / 2;
    const int NQ = NB / 4;
    const int split = blockIdx.y, splits = gridDim.y;
    const int m0 = blockIdx.z * (16 * MT);
    const int q_begin = split * QPW;
    const int nq = min(QPW, NQ - q_begin);
    const int nw = blockIdx.x * (64 * NT) + wave * (16 * NT);

    uint32_t oq[NT], os[NT], oz[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int nl = min(nw + 16 * t + c, N - 1);  // past N: re-read the last column
        oq[t] = (uint32_t)nl * (uint32_t)hk + 16u * g;
        os[t] = (uint32_t)nl * (uint32_t)NB;
        oz[t] = (uint32_t)nl * (uint32_t)(NB / 2);
    }
    // A builder role: thread = (row tid / 16 of each m-tile, slot pair tid % 16).
    // Pair kp fills dword kp % 4 of the A lane for rows 8 (kp / 4) .. + 7 of a
    // block: the activations k = 8 (kp / 4) + kp % 4 and k + 4.
    const int brow = tid >> 4, kp = tid & 15;
    const int kk = 8 * (kp >> 2) + (kp & 3);
    const bool odd = (kp & 1) != 0;
    uint32_t ox[MT];
    bool rok[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = m0 + 16 * i + brow;
        rok[i] = m < M;
        ox[i] = (uint32_t)min(m, M - 1) * (uint32_t)K + (uint32_t)kk;
    }
    const int slot = 16 * (kp >> 2) + brow;  // A lane holding this pair
    const int dw = kp & 3;                   // dword within that lane's 16 bytes

    struct Loads {
        u32x4_t w[NT];  // codes of block 4 q + g (lane group g): all 32 rows
    };
    auto issue = [&](int j, Loads &R) {
        const uint32_t q = (uint32_t)(q_begin + min(j, nq - 1));
#pragma unroll
        for (int t = 0; t < NT; ++t) R.w[t] = load_stream<u32x4_t>(Pq + (oq[t] + 64u * q));
    };

    // every quad's activations first (the build below waits for them), then
    // the first DQ quads' weights
    float2 xa[QPW][MT][4];  // (x[k], x[k + 4]) per quad, m-tile, block
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
        const uint32_t q = (uint32_t)(q_begin + min(j, nq - 1));
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float *xp = x + (ox[i] + 32u * (4u * q + b));
                xa[j][i][b] = float2{xp[0], xp[4]};
            }
    }
    // scales and zero points of all the workgroup's quads (QPW <= 4) in one
    // load each: lane (g, c) takes quad g's of column c; the quad loop reads
    // quad j's from lane (j, c)
    f32x4_t sv[NT];
    uint32_t zv[NT];
    {
        const uint32_t q = (uint32_t)(q_begin + min(g, nq - 1));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (H) {
                const u32x2_t h =
                    load_stream<u32x2_t>(static_cast<const char *>(Ps) + 2u * (os[t] + 4u * q));
                sv[t] = f32x4_t{f16_bits_to_f32((uint16_t)h.x), f16_bits_to_f32((uint16_t)(h.x >> 16)),
                                f16_bits_to_f32((uint16_t)h.y), f16_bits_to_f32((uint16_t)(h.y >> 16))};
            } else {
                sv[t] = load_stream<f32x4_t>(static_cast<const char *>(Ps) + 4u * (os[t] + 4u * q));
            }
            zv[t] = load_stream<uint16_t>(Pz + (oz[t] + 2u * q));
        }
    }
    Loads L[QPW];
#pragma unroll
    for (int j = 0; j < DQ && j < QPW; ++j) issue(j, L[j]);

    // each row's scale: max |x| over the row's activations in this workgroup's
    // K range (the row's 16 builder threads are 16 adjacent lanes)
    int sig[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        float mx = 0.0f;
#pragma unroll
        for (int j = 0; j < QPW; ++j)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (j < nq && rok[i])
                    mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fabsf(xa[j][i][b].x),
                                                             __builtin_fabsf(xa[j][i][b].y)));
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o));
        // mx = f 2^e with f in [0.5, 1): mx 2^(15 - e) lies in [2^14, 2^15)
        sig[i] = (mx > 0.0f && mx <= 3.402823466e38f) ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
        if (kp == 0) srow[i][brow] = sig[i];
    }
    // A operands: three fp16 parts of x 2^a (odd k: x 2^(a - 4))
#pragma unroll
    for (int j = 0; j < QPW; ++j)
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            uint32_t *im = reinterpret_cast<uint32_t *>(img[j][blk]);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const bool on = j < nq && rok[i];
                const int e = odd ? sig[i] - 4 : sig[i];
                const float a0 = on ? __builtin_ldexpf(xa[j][i][blk].x, e) : 0.0f;
                const float a1 = on ? __builtin_ldexpf(xa[j][i][blk].y, e) : 0.0f;
                const half2_t h = __builtin_convertvector(f32x2v{a0, a1}, half2_t);
                const float r0 = a0 - (float)h.x, r1 = a1 - (float)h.y;
                const half2_t m = __builtin_convertvector(f32x2v{r0, r1}, half2_t);
                const half2_t l = __builtin_convertvector(
                    f32x2v{r0 - (float)m.x, r1 - (float)m.y}, half2_t);
                uint32_t *base = im + ((i * 3) * 64 + slot) * 4 + dw;
                base[0] = __builtin_bit_cast(uint32_t, h);
                base[64 * 4] = __builtin_bit_cast(uint32_t, m);
                base[2 * 64 * 4] = __builtin_bit_cast(uint32_t, l);
            }
        }
    __syncthreads();

    f32x4v acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = f32x4v{0.f, 0.f, 0.f, 0.f};
    const f32x4v zero4 = {0.f, 0.f, 0.f, 0.f};
    // the code masks and the fp16 1024 pair, kept in registers for v_bfi_b32
    uint32_t mE = 0x000F000Fu, mO = 0x00F000F0u, c6400 = 0x64006400u;
    asm volatile("" : "+v"(mE), "+v"(mO), "+v"(c6400));

#pragma unroll
    for (int j = 0; j < QPW; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        if (j + DQ < QPW) issue(j + DQ, L[j + DQ]);
        __builtin_amdgcn_sched_barrier(0);
        Loads &R = L[j];
        f32x4_t sj[NT];
        uint32_t zj[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int src = j * 16 + c;
            sj[t] = f32x4_t{__shfl(sv[t].x, src), __shfl(sv[t].y, src), __shfl(sv[t].z, src),
                            __shfl(sv[t].w, src)};
            zj[t] = (uint32_t)__shfl((int)zv[t], src);
        }
        // 4 x 4 word transpose through this wave's LDS (wave-private)
        uint32_t wq[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            tq[wave][t * 64 + lane] = R.w[t];
            const uint32_t *tw = reinterpret_cast<const uint32_t *>(tq[wave] + t * 64);
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) wq[t][blk] = tw[(blk * 16 + c) * 4 + g];
        }
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            f16x8_t b[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint32_t w = wq[t][blk];
                const uint32_t zz = ((zj[t] >> (4 * blk)) & 15u) * 0x00010001u;
                const half2_t zE = as_half2(zz | 0x64006400u);         // 1024 + z
                const half2_t zO = as_half2((zz << 4) | 0x64006400u);  // 1024 + 16 z
                const uint32_t hv = w >> 8;
                const half2_t e0 = as_half2(bfi(mE, w, c6400)) - zE;   // k 0, 4
                const half2_t o0 = as_half2(bfi(mO, w, c6400)) - zO;   // k 1, 5
                const half2_t e1 = as_half2(bfi(mE, hv, c6400)) - zE;  // k 2, 6
                const half2_t o1 = as_half2(bfi(mO, hv, c6400)) - zO;  // k 3, 7
                const u32x4_t bw = {__builtin_bit_cast(uint32_t, e0), __builtin_bit_cast(uint32_t, o0),
                                    __builtin_bit_cast(uint32_t, e1), __builtin_bit_cast(uint32_t, o1)};
                b[t] = __builtin_bit_cast(f16x8_t, bw);
            }
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const u32x4_t *ai = img[j][blk] + (i * 3) * 64 + lane;
                const f16x8_t ah = __builtin_bit_cast(f16x8_t, ai[0]);
                const f16x8_t am = __builtin_bit_cast(f16x8_t, ai[64]);
                const f16x8_t al = __builtin_bit_cast(f16x8_t, ai[128]);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    f32x4v d = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, b[t], zero4, 0, 0, 0);
                    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, b[t], d, 0, 0, 0);
                    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, b[t], d, 0, 0, 0);
                    const float sc = sj[t][blk];
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[i][t][v] = __builtin_fmaf(sc, d[v], acc[i][t][v]);
                }
            }
        }
        // pin the scale-accumulate here, once per quad (see k_mm_x3)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v) asm volatile("" : "+v"(acc[i][t][v]));
    }

    // lane (g, c) holds D[4 g + v][c] of each (m-tile, column tile); the
    // tile's scale comes off here
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
                const float r = __builtin_ldexpf(acc[i][t][v], -srow[i][4 * g + v]);
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

}  // namespace

hipError_t launch_mm_x3(const X3Plan &p, const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                        const void *Ps, bool f16, const uint8_t *Pz, int64_t N, const float *bias,
                        const float *residual, int act, float *y, void *workspace,
                        hipStream_t stream) {
    const dim3 grid((unsigned)p.col_wgs, (unsigned)p.splits, (unsigned)p.mgroups);
    float *part = p.splits > 1 ? static_cast<float *>(workspace) : nullptr;
    bool launched = false;
    if (p.h3) {
#define W4_H3(QV)                                                                               \
        if (!launched && p.quads_per_wg == QV) {                                                \
            if (f16)                                                                            \
                hipLaunchKernelGGL((k_mm_h3<1, 1, QV, 3, true>), grid, dim3(256), 0, stream, x,  \
                                   (int)M, (int)K, Pq, Ps, Pz, (int)N, bias, residual, act, y,   \
                                   (int)p.npad, part);                                          \
            else                                                                                \
                hipLaunchKernelGGL((k_mm_h3<1, 1, QV, 3, false>), grid, dim3(256), 0, stream, x, \
                                   (int)M, (int)K, Pq, Ps, Pz, (int)N, bias, residual, act, y,   \
                                   (int)p.npad, part);                                          \
            launched = true;                                                                    \
        }
        W4_H3(1) W4_H3(2) W4_H3(3) W4_H3(4)
#undef W4_H3
    }
#define W4_X3(MTV, NTV, QV, DQV)                                                                \
    if (!launched && !p.h3 && p.mt == MTV && p.nt == NTV && p.quads_per_wg == QV) {                      \
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
    W4_X3_Q(1, 1, 3) W4_X3_Q(2, 1, 3) W4_X3_Q(3, 1, 2) W4_X3_Q(4, 1, 2)
    W4_X3_Q(1, 2, 3) W4_X3_Q(2, 2, 2)
#undef W4_X3_Q
#undef W4_X3
    if (!launched) return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_reduce(part, p.splits, M, N, p.npad, bias, nullptr, 1.0f, y, stream,
                                residual, act);
}

}  // namespace w4
