// K-major ("prepacked") layout of the 4-bit format, and the decode GEMV on it.
//
// The page ("ONNX export, quantization and the browser runtime", section
// "Quantization") stores each weight as a plain [K, N] UINT4 constant with a
// blocked DequantizeLinear, and mentions the runtime's weight "prepacking".
// Here prepacking is a byte-exact reordering of the same format so that the
// data of one output column is contiguous:
//   Pq uint8 [N, K/2]   codes of column n, pairs along K (low nibble = even k)
//   Ps fp32  [N, K/32]  the column's block scales
//   Pz uint8 [N, K/64]  the column's zero points, pairs of blocks per byte
// The bytes per weight are unchanged (0.640625 B).
//
// GEMV on this layout: a workgroup owns a few whole columns, so no partial
// sums leave it (no split-K across workgroups, no atomics, no workspace).
// A lane owns one 32-row block of a column: one 16-byte load of codes, one
// scale, one zero point, and the 32 activations of that block (held in
// registers across all the workgroup's columns).  64 lanes read 1 KB of one
// column contiguously.  Per packed word: 1 shift, 4 masks, 4 packed-fp16
// subtractions (q - z as exact fp16 subnormals) and 8 v_fma_mix_f32.  The
// per-lane block sums are scaled, then summed over the column's lanes in a
// fixed order: where every 32-lane half of a wave lies in one column slot
// (K a multiple of 1024), each half adds its lanes in registers (DPP) and one
// value per half crosses LDS; otherwise all lane partials go through LDS, a
// few lanes per output each adding a contiguous run, then two lane
// exchanges.  Results are deterministic.
#include <type_traits>

#include "common.h"
#include "epilogue.h"
#include "launch.h"

namespace w4 {
namespace {

// Relayout, one thread per (column pair j, k pair i): reads the two packed
// bytes Wq[2i, j], Wq[2i+1, j] (columns 2j, 2j+1) and writes Pq[2j, i] and
// Pq[2j+1, i].  Consecutive threads take consecutive i (coalesced writes).
__global__ __launch_bounds__(256) void k_prepack_codes(const uint8_t *__restrict__ Wq, int64_t K,
                                                       int64_t N, uint8_t *__restrict__ Pq) {
    const int64_t hk = K / 2, half = N / 2;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= hk * half) return;
    const int64_t j = t / hk, i = t - j * hk;
    const uint8_t a = Wq[(2 * i) * half + j];      // row 2i: columns 2j (low), 2j+1 (high)
    const uint8_t b = Wq[(2 * i + 1) * half + j];  // row 2i+1
    Pq[(2 * j) * hk + i] = (uint8_t)((a & 15) | ((b & 15) << 4));
    Pq[(2 * j + 1) * hk + i] = (uint8_t)((a >> 4) | (b & 0xF0));
}

// Scales and zero points, one thread per (column pair j, block pair c).
template <bool H>
__global__ __launch_bounds__(256) void k_prepack_blocks(const void *__restrict__ scales_v,
                                                        const uint8_t *__restrict__ zeros,
                                                        int64_t K, int64_t N,
                                                        void *__restrict__ Ps_v,
                                                        uint8_t *__restrict__ Pz) {
    typedef typename std::conditional<H, uint16_t, float>::type S;  // scale storage
    const S *scales = static_cast<const S *>(scales_v);
    S *Ps = static_cast<S *>(Ps_v);
    const int64_t NB = K / kBlock, half = N / 2, hb = NB / 2;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= hb * half) return;
    const int64_t j = t / hb, c = t - j * hb;
    const int64_t b0 = 2 * c, b1 = 2 * c + 1;
    const uint8_t z0 = zeros[b0 * half + j], z1 = zeros[b1 * half + j];
    Pz[(2 * j) * hb + c] = (uint8_t)((z0 & 15) | ((z1 & 15) << 4));
    Pz[(2 * j + 1) * hb + c] = (uint8_t)((z0 >> 4) | (z1 & 0xF0));
    Ps[(2 * j) * NB + b0] = scales[b0 * N + 2 * j];
    Ps[(2 * j) * NB + b1] = scales[b1 * N + 2 * j];
    Ps[(2 * j + 1) * NB + b0] = scales[b0 * N + 2 * j + 1];
    Ps[(2 * j + 1) * NB + b1] = scales[b1 * N + 2 * j + 1];
}

// Sum of v over each 32-lane half of the wave, in DPP steps (no LDS): pairs,
// quads, rotations by 4 and 8 within each 16-lane row, then row 0 (2) into
// row 1 (3).  The sums are valid in lanes 31 and 63; the order of the
// additions is fixed, so the result does not depend on timing.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                   0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float sum32(float v) {
    v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x124, 0xF>(v);  // row_ror:4
    v = dpp_add<0x128, 0xF>(v);  // row_ror:8
    v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    return v;
}

// acc[r] += x_r[k] * (q[k] - z) over the 16 codes k = 16h .. 16h+15 of two
// consecutive words (v0: k = 16h .. 16h+7, v1: the next 8), for MR
// activation rows.  One 64-bit shift serves both words: the masks below only
// read bits 0-7 and 16-23 of each 32-bit half, which the shift fills from
// the right word.  Even k land in accE (units 2^-24), odd k in accO (units
// 2^-20); see common.h for the subnormal encoding.
template <int MR>
__device__ __forceinline__ void fma_kpair(uint32_t v0, uint32_t v1, half2_t zE, half2_t zO,
                                          const float (*xr)[kBlock], int h, float *accE,
                                          float *accO) {
    const uint64_t sh = (((uint64_t)v1 << 32) | v0) >> 8;
    const uint32_t hv[2] = {(uint32_t)sh, (uint32_t)(sh >> 32)};
    const uint32_t lv[2] = {v0, v1};
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const half2_t e0 = as_half2(lv[d] & 0x000F000Fu) - zE;  // k = +0, +4
        const half2_t o0 = as_half2(lv[d] & 0x00F000F0u) - zO;  // k = +1, +5
        const half2_t e1 = as_half2(hv[d] & 0x000F000Fu) - zE;  // k = +2, +6
        const half2_t o1 = as_half2(hv[d] & 0x00F000F0u) - zO;  // k = +3, +7
        const int k = 16 * h + 8 * d;
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            accE[r] = __builtin_fmaf(xr[r][k + 0], (float)e0.x, accE[r]);
            accO[r] = __builtin_fmaf(xr[r][k + 1], (float)o0.x, accO[r]);
            accE[r] = __builtin_fmaf(xr[r][k + 2], (float)e1.x, accE[r]);
            accO[r] = __builtin_fmaf(xr[r][k + 3], (float)o1.x, accO[r]);
            accE[r] = __builtin_fmaf(xr[r][k + 4], (float)e0.y, accE[r]);
            accO[r] = __builtin_fmaf(xr[r][k + 5], (float)o0.y, accO[r]);
            accE[r] = __builtin_fmaf(xr[r][k + 6], (float)e1.y, accE[r]);
            accO[r] = __builtin_fmaf(xr[r][k + 7], (float)o1.y, accO[r]);
        }
    }
}

// One workgroup: columns n0 .. n0 + CC - 1 (CC = G * P), MR rows of x
// starting at row m0 = blockIdx.y * MR.  The arguments that the first loads
// depend on come first: they fit the 14 kernel-argument registers the
// hardware fills at wave launch (the library is built with kernel-argument
// preloading), so no wave waits for an argument load before its first
// weight load; bias, residual, act and y are read only at the end.  Lane L = (g, bl): column slot
// g = L / NBL and block bl, then bl + NBL, ... while < NB.  Pass p covers
// column n0 + p * G + g.  Offsets are 32-bit (the host keeps every array
// below 2^31 bytes).  CHECK clamps columns past N (ragged last workgroup);
// without it every load is unconditional, so the compiler can start on
// pass 0 while later passes are still in flight.
// AFF: the group-64 affine variant, Ps = scales and Pz = minima, fp32
// [N, K/64]: a lane's block is half a group, and its sum is
// s * sum_k x q + m * sum_k x, with sum_k x formed once per lane and reused
// by every pass (the codes enter as the same fp16 subnormals, unshifted).
// XC (one or two rows, NBL == NB so every lane owns exactly one block,
// NBL % 8 == 0, every lane in a column slot): the activations are read
// in whole 1 KB runs: load instruction i reads the 8 consecutive blocks that
// lane group i of the wave owns, lane l taking bytes 16 (l % 8) of the run's
// block l / 8; wave-private LDS (144-byte block slots, so the 16-byte reads
// of one block per lane do not collide) then hands every lane its own
// block.  A lane's own block's 128 bytes would otherwise come from 8 loads
// that each touch 64 different cache lines.
// XC selects how the activations arrive: kXcLane (0) each lane loads its own
// block, kXcRuns (1) the wave runs above, kXcShared + G (G column slots per
// workgroup, NBL == NB; G = 2 is instantiated): the slots need the same
// activations, so the workgroup reads each row once in coalesced 16-byte
// chunks (thread t takes chunks t, t + T, t + 2T and t + 3T of the row, T
// threads), stages it in LDS in 144-byte block slots, and one barrier hands
// every lane its block.  The barrier's fence covers LDS only: a full
// workgroup fence would wait for every weight load still in flight, and all
// arithmetic would wait for the last of them.  It halves the activation
// traffic of the wave runs (3.8B shapes, us per launch: 3072 x 9216 6.10 ->
// 5.62, 3072 x 16384 8.09 -> 7.89, 3072 x 3072 3.72 -> 3.60, with the
// passes chosen for it).
// NBLC: NBL as a compile-time constant (0: the argument).  The lane's slot
// and the activation runs' blocks come from divisions by NBL before the first
// weight load; by a constant they are a multiply and a shift (3.8B M=1 pass:
// 101 -> 51..66 instructions before the first load, 0.763 -> 0.728 ms).
constexpr int kXcLane = 0, kXcRuns = 1, kXcShared = 16;
template <int MR, int P, bool CHECK, int LM, bool H, bool EP, bool AFF = false,
          int XC = kXcLane, int NBLC = 0>
__global__ __launch_bounds__(256) void k_gemv_kmajor(
    const float *__restrict__ x, const uint8_t *__restrict__ Pq, const void *__restrict__ Ps,
    const void *__restrict__ Pz, int M, int K, int N, int G, int NBL_arg,
    const float *__restrict__ bias, const float *residual, int act, float *y) {
    extern __shared__ float red[];  // [MR][CC][NBL]; XC: then 36 floats per lane
    const int NBL = NBLC ? NBLC : NBL_arg;
    const int L = threadIdx.x;
    const int g = L / NBL, bl = L - g * NBL;
    const int NB = K / kBlock, hk = K / 2;
    const int CC = G * P;
    const int n0 = blockIdx.x * CC;
    const int m0 = blockIdx.y * MR;

    float part[MR][P];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int p = 0; p < P; ++p) part[r][p] = 0.0f;

    if (g < G) {
        // LM != 1: NBL >= NB, each lane owns at most one block (no loop)
        for (int b = bl; LM == 1 ? b < NB : (b == bl && b < NB); b += NBL) {
            // activations of this block, for each of the MR rows
            float xr[MR][kBlock];
            constexpr bool RUNS = XC == kXcRuns, SHARED = XC > kXcShared;
            f32x4_t xg[RUNS ? MR : 1][RUNS ? kBlock / 4 : 1];  // 16 bytes of each of 8 runs
            constexpr int XG = SHARED ? XC - kXcShared : 1;    // column slots sharing the rows
            constexpr int XW = SHARED ? kBlock / 4 / XG : 1;   // chunks per thread and row
            f32x4_t xw[SHARED ? MR : 1][XW];
            const int lw = L & 63;
            if (SHARED) {
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    const float *xrow = x + (size_t)min(m0 + r, M - 1) * K;
#pragma unroll
                    for (int i = 0; i < XW; ++i)
                        xw[r][i] = *reinterpret_cast<const f32x4_t *>(xrow + 4 * (L + i * XG * NBL));
                }
            }
            if (RUNS) {
                // run i: the 8 blocks of lane group i of this wave, from block
                // bl(8 i); this lane takes block lw / 8 of it, bytes 16 (lw % 8)
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    const float *xrow = x + (size_t)min(m0 + r, M - 1) * K;
#pragma unroll
                    for (int i = 0; i < kBlock / 4; ++i) {
                        const int li = (L & ~63) + 8 * i;
                        const int bi = li - (li / NBL) * NBL;
                        xg[r][i] = *reinterpret_cast<const f32x4_t *>(
                            xrow + kBlock * (bi + (lw >> 3)) + 4 * (lw & 7));
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < (XC != kXcLane ? 0 : MR); ++r) {
                const int m = min(m0 + r, M - 1);
                const f32x4_t *xp = reinterpret_cast<const f32x4_t *>(x + (size_t)m * K + b * kBlock);
#pragma unroll
                for (int i = 0; i < kBlock / 4; ++i) {
                    const f32x4_t v = xp[i];
                    xr[r][4 * i + 0] = v.x;
                    xr[r][4 * i + 1] = v.y;
                    xr[r][4 * i + 2] = v.z;
                    xr[r][4 * i + 3] = v.w;
                }
            }
            // codes, scale and zero point (or minimum) of this block, for each
            // pass's column
            u32x4_t w[P];
            float s[P], mn[P];
            uint32_t zb[P];
            const int nf = n0 + g;  // this lane's column in pass 0
            const int NS = AFF ? NB / 2 : NB;  // scales per column
            const int bs = AFF ? (b >> 1) : b;
            uint32_t oq = (uint32_t)(nf * hk + 16 * b);
            uint32_t os = (uint32_t)(nf * NS + bs);
            uint32_t oz = (uint32_t)(nf * (NB / 2) + (b >> 1));
            const uint32_t sq = (uint32_t)(G * hk), ss = (uint32_t)(G * NS),
                           sz = (uint32_t)(G * (NB / 2));
#pragma unroll
            for (int p = 0; p < P; ++p) {
                uint32_t q_off = oq, s_off = os, z_off = oz;
                if (CHECK && n0 + p * G + g >= N) {  // past the last column: re-read it
                    const int nl = N - 1;
                    q_off = (uint32_t)(nl * hk + 16 * b);
                    s_off = (uint32_t)(nl * NS + bs);
                    z_off = (uint32_t)(nl * (NB / 2) + (b >> 1));
                }
                w[p] = load_stream<u32x4_t>(Pq + q_off);
                // scales and zero points are read once, like the codes: streaming
                // loads (3.8B M=1 pass 0.842 -> 0.818 ms against plain loads)
                s[p] = H ? f16_bits_to_f32(load_stream<uint16_t>(static_cast<const uint16_t *>(Ps) + s_off))
                         : load_stream<float>(static_cast<const float *>(Ps) + s_off);
                if (AFF) {
                    mn[p] = load_stream<float>(static_cast<const float *>(Pz) + s_off);
                    zb[p] = 0;
                } else {
                    mn[p] = 0.0f;
                    zb[p] = load_stream<uint8_t>(static_cast<const uint8_t *>(Pz) + z_off);
                }
                oq += sq;
                os += ss;
                oz += sz;
            }
            __builtin_amdgcn_sched_barrier(0);  // every load in flight before the arithmetic
            if (SHARED) {
                // chunk c of row r to piece c % 8 of block slot c / 8
                float *xs = red + MR * CC * NBL;
#pragma unroll
                for (int r = 0; r < MR; ++r)
#pragma unroll
                    for (int i = 0; i < XW; ++i) {
                        const int c = L + i * XG * NBL;
                        *reinterpret_cast<f32x4_t *>(xs + 36 * (r * NBL + (c >> 3)) + 4 * (c & 7)) = xw[r][i];
                    }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
                for (int r = 0; r < MR; ++r)
#pragma unroll
                    for (int i = 0; i < kBlock / 4; ++i) {
                        const f32x4_t v =
                            *reinterpret_cast<const f32x4_t *>(xs + 36 * (r * NBL + bl) + 4 * i);
                        xr[r][4 * i + 0] = v.x;
                        xr[r][4 * i + 1] = v.y;
                        xr[r][4 * i + 2] = v.z;
                        xr[r][4 * i + 3] = v.w;
                    }
            }
            if (RUNS) {
                // run i's pieces to block slot 8 i + lw / 8 of this wave's
                // staging area; then this lane's own block is slot lw
                float *xstage = red + MR * CC * NBL + (L & ~63) * (36 * MR);
#pragma unroll
                for (int r = 0; r < MR; ++r)
#pragma unroll
                    for (int i = 0; i < kBlock / 4; ++i)
                        *reinterpret_cast<f32x4_t *>(xstage + 36 * (64 * r + 8 * i + (lw >> 3)) +
                                                     4 * (lw & 7)) = xg[r][i];
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int r = 0; r < MR; ++r)
#pragma unroll
                    for (int i = 0; i < kBlock / 4; ++i) {
                        const f32x4_t v =
                            *reinterpret_cast<const f32x4_t *>(xstage + 36 * (64 * r + lw) + 4 * i);
                        xr[r][4 * i + 0] = v.x;
                        xr[r][4 * i + 1] = v.y;
                        xr[r][4 * i + 2] = v.z;
                        xr[r][4 * i + 3] = v.w;
                    }
            }
            float xs[MR];  // AFF: sum of the block's activations, per row
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                xs[r] = 0.0f;
                if (AFF) {
#pragma unroll
                    for (int k = 0; k < kBlock; ++k) xs[r] += xr[r][k];
                }
            }
            const int zsh = (b & 1) * 4;
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const uint32_t z = AFF ? 0u : (zb[p] >> zsh) & 15;  // AFF: codes as they are
                const half2_t zE = as_half2(z * 0x00010001u);
                const half2_t zO = as_half2((z << 4) * 0x00010001u);
                float accE[MR], accO[MR];
#pragma unroll
                for (int r = 0; r < MR; ++r) accE[r] = accO[r] = 0.0f;
                fma_kpair<MR>(w[p].x, w[p].y, zE, zO, xr, 0, accE, accO);
                fma_kpair<MR>(w[p].z, w[p].w, zE, zO, xr, 1, accE, accO);
#pragma unroll
                for (int r = 0; r < MR; ++r) {
                    const float t = __builtin_fmaf(accO[r], 1048576.0f, accE[r] * 16777216.0f);
                    if (AFF)
                        part[r][p] = __builtin_fmaf(s[p], t, __builtin_fmaf(mn[p], xs[r], part[r][p]));
                    else
                        part[r][p] = __builtin_fmaf(s[p], t, part[r][p]);
                }
                // Keep each pass's arithmetic here, in load order, so that it
                // waits only for its own data: the partial sums are read only
                // by the reduction below, and the compiler would otherwise sink
                // every pass's FMAs there, behind the last load.  An empty asm
                // that reads and writes each partial pins them in place; the
                // scheduling barrier keeps later passes' unpacking out of it.
#pragma unroll
                for (int r = 0; r < MR; ++r) asm volatile("" : "+v"(part[r][p]));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    if (LM == 2) {
        // Every 32-lane half belongs to one column slot (slots start at
        // multiples of NBL): each half sums its partials in registers, and
        // only one value per half and output goes through LDS, [MR][CC][NHV].
        // 3.8B M=1 pass 0.817 -> 0.763 ms against the LDS sum of all lanes.
        const int NHV = NBL >> 5;
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
            for (int p = 0; p < P; ++p) part[r][p] = sum32(part[r][p]);
        if (NBLC == 32) {
            // Each column slot is one 32-lane half (lanes past the column's
            // blocks idle): its last lane holds the column's sum and stores
            // it; no LDS and no barrier.  A SwiGLU pair (c, c + 1), c even, is
            // slots g and g + 1 (G is even), the two halves of one wave.
            float up[MR][P];
#pragma unroll
            for (int r = 0; r < MR; ++r)
#pragma unroll
                for (int p = 0; p < P; ++p) up[r][p] = __shfl_down(part[r][p], 32);
            if (g < G && bl == 31) {
#pragma unroll
                for (int r = 0; r < MR; ++r)
#pragma unroll
                    for (int p = 0; p < P; ++p) {
                        const int n = n0 + p * G + g, m = m0 + r;
                        if (n >= N || m >= M) continue;
                        float v = part[r][p];
                        if (EP) {
                            if (bias) v += bias[n];
                            if (act == W4_ACT_SWIGLU) {
                                if ((g & 1) == 0) {
                                    const float u = up[r][p] + (bias ? bias[n + 1] : 0.0f);
                                    ep_store_glu(v, u, residual, y, (size_t)m * (N / 2) + n / 2);
                                }
                            } else {
                                ep_store(v, act, residual, y, (size_t)m * N + n);
                            }
                        } else {
                            y[(size_t)m * N + n] = bias ? v + bias[n] : v;
                        }
                    }
            }
            return;
        }
        if (g < G && (bl & 31) == 31) {
#pragma unroll
            for (int r = 0; r < MR; ++r)
#pragma unroll
                for (int p = 0; p < P; ++p) red[(r * CC + p * G + g) * NHV + (bl >> 5)] = part[r][p];
        }
        __syncthreads();
        for (int o = L; o < MR * CC; o += blockDim.x) {
            float v = red[o * NHV];
            for (int h = 1; h < NHV; ++h) v += red[o * NHV + h];
            const int r = MR == 1 ? 0 : o / CC, c = o - r * CC;
            const int n = n0 + c, m = m0 + r;
            if (n >= N || m >= M) continue;
            if (EP) {
                if (bias) v += bias[n];
                if (act == W4_ACT_SWIGLU) {
                    // CC is even: column pair (c, c + 1), c even, is outputs o and o + 1
                    if ((c & 1) == 0) {
                        float up = red[(o + 1) * NHV];
                        for (int h = 1; h < NHV; ++h) up += red[(o + 1) * NHV + h];
                        if (bias) up += bias[n + 1];
                        ep_store_glu(v, up, residual, y, (size_t)m * (N / 2) + n / 2);
                    }
                } else {
                    ep_store(v, act, residual, y, (size_t)m * N + n);
                }
            } else {
                y[(size_t)m * N + n] = bias ? v + bias[n] : v;
            }
        }
        return;
    }

    // lane partials -> LDS as [MR][CC][NBL]; column c = p * G + g
    if (g < G) {
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
            for (int p = 0; p < P; ++p) red[(r * CC + p * G + g) * NBL + bl] = part[r][p];
    }
    __syncthreads();
    // `parts` adjacent lanes per output each add one contiguous run of NBL /
    // parts partials in order, then the runs are added by two lane exchanges:
    // a fixed order, so the result does not depend on timing.
    const int parts = (NBL % 4 == 0) ? 4 : ((NBL % 2 == 0) ? 2 : 1);
    const int per = NBL / parts;
    const int q = L % parts;
    for (int o = L / parts; o < MR * CC; o += blockDim.x / parts) {
        const float *rp = red + o * NBL + q * per;
        float v = 0.0f;
        if ((per & 3) == 0) {  // 16-byte aligned runs: vector reads, pairwise adds
            for (int j = 0; j < per; j += 4) {
                const f32x4_t t = *reinterpret_cast<const f32x4_t *>(rp + j);
                v += (t.x + t.y) + (t.z + t.w);
            }
        } else {
            for (int j = 0; j < per; ++j) v += rp[j];
        }
        if (parts >= 2) v += __shfl_xor(v, 1);
        if (parts == 4) v += __shfl_xor(v, 2);
        const int r = o / CC, c = o - r * CC;
        const int n = n0 + c, m = m0 + r;
        if (EP) {  // the fused epilogue, in its own instantiation
            if (bias && n < N) v += bias[n];
            if (act == W4_ACT_SWIGLU) {
                // CC is even, so column pair (c, c + 1), c even, is outputs o
                // and o + 1: the next group of `parts` lanes, same wave and round
                const float up = __shfl_down(v, parts);
                if (q == 0 && (c & 1) == 0 && n < N && m < M)
                    ep_store_glu(v, up, residual, y, (size_t)m * (N / 2) + n / 2);
            } else if (q == 0 && n < N && m < M) {
                ep_store(v, act, residual, y, (size_t)m * N + n);
            }
        } else if (q == 0 && n < N && m < M) {
            y[(size_t)m * N + n] = bias ? v + bias[n] : v;
        }
    }
}

// K = 0: every pre-activation value is the bias (or 0); the epilogue alone,
// one thread per output.
__global__ __launch_bounds__(256) void k_epilogue_only(const float *__restrict__ bias, int64_t M,
                                                       int64_t N,
                                                       const float *residual, int act,
                                                       float *y) {
    const int64_t nout = act == W4_ACT_SWIGLU ? N / 2 : N;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= M * nout) return;
    const int64_t j = i - (i / nout) * nout;
    if (act == W4_ACT_SWIGLU)
        ep_store_glu(bias ? bias[2 * j] : 0.0f, bias ? bias[2 * j + 1] : 0.0f, residual, y, i);
    else
        ep_store(bias ? bias[j] : 0.0f, act, residual, y, i);
}

// Group-64 affine variant: scales and minima [K/64, N] -> [N, K/64], one
// thread per (column n, group c); consecutive threads take consecutive c.
__global__ __launch_bounds__(256) void k_prepack_g64(const float *__restrict__ scales,
                                                     const float *__restrict__ mins, int64_t K,
                                                     int64_t N, float *__restrict__ Ps,
                                                     float *__restrict__ Pm) {
    const int64_t NG = K / 64;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= NG * N) return;
    const int64_t n = t / NG, c = t - n * NG;
    Ps[t] = scales[c * N + n];
    Pm[t] = mins[c * N + n];
}

}  // namespace

hipError_t launch_prepack_g64(const uint8_t *Wq, const float *scales, const float *mins,
                              int64_t K, int64_t N, uint8_t *Pq, float *Ps, float *Pm,
                              hipStream_t stream) {
    const int64_t t1 = (K / 2) * (N / 2), t2 = (K / 64) * N;
    if (t1 > 0)
        hipLaunchKernelGGL(k_prepack_codes, dim3((unsigned)((t1 + 255) / 256)), dim3(256), 0, stream,
                           Wq, K, N, Pq);
    if (t2 > 0)
        hipLaunchKernelGGL(k_prepack_g64, dim3((unsigned)((t2 + 255) / 256)), dim3(256), 0, stream,
                           scales, mins, K, N, Ps, Pm);
    return hipGetLastError();
}

hipError_t launch_epilogue_only(const float *bias, int64_t M, int64_t N, const float *residual,
                                int act, float *y, hipStream_t stream) {
    const int64_t total = M * (act == W4_ACT_SWIGLU ? N / 2 : N);
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(k_epilogue_only, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, bias, M, N, residual, act, y);
    return hipGetLastError();
}

hipError_t launch_prepack_kmajor(const uint8_t *Wq, const void *scales, bool f16,
                                 const uint8_t *zeros, int64_t K, int64_t N, uint8_t *Pq, void *Ps,
                                 uint8_t *Pz, hipStream_t stream) {
    const int64_t t1 = (K / 2) * (N / 2), t2 = (K / 64) * (N / 2);
    if (t1 > 0)
        hipLaunchKernelGGL(k_prepack_codes, dim3((unsigned)((t1 + 255) / 256)), dim3(256), 0, stream,
                           Wq, K, N, Pq);
    if (t2 > 0) {
        const dim3 grid((unsigned)((t2 + 255) / 256));
        if (f16)
            hipLaunchKernelGGL(k_prepack_blocks<true>, grid, dim3(256), 0, stream, scales, zeros, K,
                               N, Ps, Pz);
        else
            hipLaunchKernelGGL(k_prepack_blocks<false>, grid, dim3(256), 0, stream, scales, zeros, K,
                               N, Ps, Pz);
    }
    return hipGetLastError();
}

hipError_t launch_gemv_kmajor(const KmajorPlan &p, const float *x, int64_t M, int64_t K,
                              const uint8_t *Pq, const void *Ps, bool f16, const void *Pz,
                              int64_t N, const float *bias, const float *residual, int act,
                              float *y, hipStream_t stream, bool affine) {
    if (p.kind == KmajorPlan::kEmpty) return hipSuccess;
    if (p.kind == KmajorPlan::kBiasOnly) {
        if (act == W4_ACT_NONE && !residual) return launch_bias_fill(bias, M, N, y, stream);
        return launch_epilogue_only(bias, M, N, residual, act, y, stream);
    }
    const int64_t C = (int64_t)p.groups * p.passes;
    const dim3 grid((unsigned)((N + C - 1) / C), (unsigned)((M + p.rows - 1) / p.rows));
    const bool check = (N % C) != 0;
    // lane mode: 1 = lanes loop over blocks; else one block per lane, and 2
    // when every 32-lane half of a wave lies in one column slot (its partial
    // sums are added in registers before the cross-wave step)
    const bool loop = p.lanes_per_col < K / kBlock;
    const int lm = loop ? 1 : (p.lanes_per_col % 32 == 0 ? 2 : 0);
    // whole-run activation loads: one or two rows, exactly one block per lane (no
    // idle lanes: every lane of a wave takes part in the runs' loads), 8-lane
    // groups inside one column slot
    const bool xc = p.xc && p.rows <= 2 && p.lanes_per_col == K / kBlock &&
                    p.lanes_per_col % 8 == 0 && (int64_t)p.groups * p.lanes_per_col == p.threads;
    // workgroup-shared activations: two column slots of one block per lane
    // (LDS holds one 144-byte slot per block and row)
    const bool xs = xc && p.xs == 2 && p.groups == 2;
    const size_t shm = (size_t)p.rows * C * p.lanes_per_col * sizeof(float) +
                       (xs ? (size_t)p.lanes_per_col * 36 * p.rows * sizeof(float)
                           : xc ? (size_t)p.threads * 36 * p.rows * sizeof(float) : 0);
    const bool ep = act != W4_ACT_NONE || residual;  // fp32 scales only (checked by the caller)
#define W4_KM_ARGS                                                                              \
    x, Pq, Ps, Pz, (int)M, (int)K, (int)N, p.groups, p.lanes_per_col, bias, residual, act, y
#define W4_KM_LAUNCH2(MRV, PV, CV, LV, XCV, NV)                                                     \
    if (affine)                                                                                     \
        hipLaunchKernelGGL((k_gemv_kmajor<MRV, PV, CV, LV, false, false, true, XCV, NV>), grid,   \
                           dim3(p.threads), shm, stream, W4_KM_ARGS);                           \
    else if (f16)                                                                                   \
        hipLaunchKernelGGL((k_gemv_kmajor<MRV, PV, CV, LV, true, false, false, XCV, NV>), grid,   \
                           dim3(p.threads), shm, stream, W4_KM_ARGS);                           \
    else if (ep)                                                                                    \
        hipLaunchKernelGGL((k_gemv_kmajor<MRV, PV, CV, LV, false, true, false, XCV, NV>), grid,   \
                           dim3(p.threads), shm, stream, W4_KM_ARGS);                           \
    else                                                                                            \
        hipLaunchKernelGGL((k_gemv_kmajor<MRV, PV, CV, LV, false, false, false, XCV, NV>), grid,  \
                           dim3(p.threads), shm, stream, W4_KM_ARGS)
// Constant-NBL instantiations: one or two rows with whole-run activation
// loads and 96 or 256 lanes per column (the 3.8B shapes' K = 3072 and 8192);
// and one or two rows with 32 lanes per column (K = 544 .. 1024), whose
// column sums stay in registers and are stored by one lane of each half.
#define W4_KM_LAUNCH(MRV, PV, CV, LV)                                                               \
    if (MRV <= 2 && LV != 1 && xc) {                                                                \
        if constexpr (MRV == 1 && LV == 2) {                                                        \
            if (xs && p.lanes_per_col == 96) { W4_KM_LAUNCH2(MRV, PV, CV, LV, kXcShared + 2, 96); } \
            else if (p.lanes_per_col == 96) { W4_KM_LAUNCH2(MRV, PV, CV, LV, kXcRuns, 96); }        \
            else if (p.lanes_per_col == 256) { W4_KM_LAUNCH2(MRV, PV, CV, LV, kXcRuns, 256); }      \
            else if (p.lanes_per_col == 32) { W4_KM_LAUNCH2(MRV, PV, CV, LV, kXcRuns, 32); }        \
            else { W4_KM_LAUNCH2(MRV, PV, CV, LV, kXcRuns, 0); }                                    \
        } else if constexpr (MRV == 2 && LV == 2) {                                                 \
            if (xs && p.lanes_per_col == 96) { W4_KM_LAUNCH2(MRV, PV, CV, LV, kXcShared + 2, 96); } \
            else if (p.lanes_per_col == 32) { W4_KM_LAUNCH2(MRV, PV, CV, LV, kXcRuns, 32); }        \
            else if (p.lanes_per_col == 96) { W4_KM_LAUNCH2(MRV, PV, CV, LV, kXcRuns, 96); }        \
            else if (p.lanes_per_col == 256) { W4_KM_LAUNCH2(MRV, PV, CV, LV, kXcRuns, 256); }      \
            else { W4_KM_LAUNCH2(MRV, PV, CV, LV, kXcRuns, 0); }                                    \
        } else {                                                                                    \
            W4_KM_LAUNCH2(MRV, PV, CV, LV, MRV <= 2 && LV != 1 ? kXcRuns : kXcLane, 0);             \
        }                                                                                           \
    } else {                                                                                        \
        if constexpr (MRV <= 2 && LV == 2) {                                                        \
            if (p.lanes_per_col == 32) { W4_KM_LAUNCH2(MRV, PV, CV, LV, kXcLane, 32); }             \
            else { W4_KM_LAUNCH2(MRV, PV, CV, LV, kXcLane, 0); }                                    \
        } else {                                                                                    \
            W4_KM_LAUNCH2(MRV, PV, CV, LV, kXcLane, 0);                                             \
        }                                                                                           \
    }
#define W4_KM_CASE(MRV, PV)                                                                     \
    if (p.rows == MRV && p.passes == PV) {                                                          \
        if (check) {                                                                                \
            if (lm == 1) { W4_KM_LAUNCH(MRV, PV, true, 1); }                                        \
            else if (lm == 2) { W4_KM_LAUNCH(MRV, PV, true, 2); }                                   \
            else { W4_KM_LAUNCH(MRV, PV, true, 0); }                                                \
        } else {                                                                                    \
            if (lm == 1) { W4_KM_LAUNCH(MRV, PV, false, 1); }                                       \
            else if (lm == 2) { W4_KM_LAUNCH(MRV, PV, false, 2); }                                  \
            else { W4_KM_LAUNCH(MRV, PV, false, 0); }                                               \
        }                                                                                           \
        return hipGetLastError();                                                               \
    }
    W4_KM_CASE(1, 1) W4_KM_CASE(1, 2) W4_KM_CASE(1, 3) W4_KM_CASE(1, 4)
    W4_KM_CASE(1, 6) W4_KM_CASE(1, 8) W4_KM_CASE(1, 12) W4_KM_CASE(1, 16)
    W4_KM_CASE(2, 1) W4_KM_CASE(2, 2) W4_KM_CASE(2, 4)
    W4_KM_CASE(4, 1) W4_KM_CASE(4, 2)
#undef W4_KM_ARGS
#undef W4_KM_LAUNCH
#undef W4_KM_LAUNCH2
#undef W4_KM_CASE
    return hipErrorInvalidValue;
}

}  // namespace w4
