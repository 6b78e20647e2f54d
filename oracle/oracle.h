/*
 * CPU oracle for the 4-bit block-dequant weight matmul and the int8 tied LM head.
 *
 * TEST INFRASTRUCTURE ONLY.  This code exists to check the HIP library; it is
 * never part of the product path.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header, table or
 * helper with the HIP library and includes nothing from it.
 *
 * Source of the method: the page "ONNX export, quantization and the browser
 * runtime", section "Quantization (train/quantize.py)", steps 1-4:
 *   - each linear layer of the body is a [K, N] weight matrix and a bias;
 *   - the matrix is kept in 4 bits: in every column each run of 32 rows is
 *     quantized asymmetrically with its own scale (fp32) and zero point
 *     (uint4), the codes are packed two to a byte, and dequantization gives
 *     back fp32 values;
 *   - the embedding and the LM head share a single int8 table laid out as
 *     [768, 50257], with an fp32 scale for each token;
 *   - logits are needed for the final position alone.
 * The same page, paragraph after the steps: the runtime folds the dequantize
 * nodes and runs plain fp32 kernels, so the matmul computes x . W_hat with
 * W_hat the fp32 output of the dequantization.
 *
 * Readings where the page is silent: pairs of nibbles run along N (flat
 * row-major packing of the [K, N] code tensor, element 2i in the low nibble);
 * the block range includes 0; rounding is IEEE round-half-to-even; scale,
 * zero and code arithmetic is fp32 with no contraction; accumulation is fp64
 * with one final rounding.
 *
 * Every function is plain loops, no blocking, no fusion; status 0 = OK.
 */
#ifndef W4_ORACLE_H
#define W4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ORC_OK = 0,
    ORC_BAD_SHAPE = 1, /* K % 32 != 0, N odd, negative size, ldq < N      */
    ORC_NONFINITE = 2, /* a non-finite weight, or a scale that overflowed */
    ORC_NO_MEMORY = 3  /* malloc failed                                    */
};

/* Threads shared among a call's independent outputs (OpenMP; 0 or less
 * leaves the setting unchanged), and the current count.  Results do not
 * depend on it.                                                              */
void orc_set_threads(int n);
int orc_get_threads(void);

/* Pack count (even) 4-bit values, one per byte in v[0..count), two per byte:
 * out[i] = v[2i] | v[2i+1] << 4 (the low nibble holds the even element).     */
void orc_pack_u4(const uint8_t *v, int64_t count, uint8_t *out);

/* Inverse of orc_pack_u4: v[2i] = in[i] & 15, v[2i+1] = in[i] >> 4.          */
void orc_unpack_u4(const uint8_t *in, int64_t count, uint8_t *v);

/* Block quantizer (page section "Quantization", step 2).
 * W      fp32 [K, N] row-major, K % 32 == 0, N even.
 * Wq     uint8 [K, N/2]: packed codes q[k, n], pairs along n.
 * scales fp32 [K/32, N]: scale of block b = rows 32b..32b+31 of column n.
 * zeros  uint8 [K/32, N/2]: packed zero points z[b, n], pairs along n.
 * Per block: lo = min(0, min w), hi = max(0, max w); s = (hi - lo) / 15;
 * s == 0 gives s = z = q = 0; z = clamp(rint(-lo / s), 0, 15);
 * q = clamp(rint(w / s) + z, 0, 15).                                        */
int orc_w4_quantize_pack(const float *W, int64_t K, int64_t N,
                         uint8_t *Wq, float *scales, uint8_t *zeros);

/* Unpack codes and zero points: q uint8 [K, N], z uint8 [K/32, N].         */
int orc_w4_unpack(const uint8_t *Wq, const uint8_t *zeros, int64_t K, int64_t N,
                  uint8_t *q, uint8_t *z);

/* Blocked dequantization: W_hat[k, n] = fl32((q[k, n] - z[k/32, n]) * s[k/32, n]). */
int orc_w4_dequantize(const uint8_t *Wq, const float *scales, const uint8_t *zeros,
                      int64_t K, int64_t N, float *W_hat);

/* K-major relayout of the 4-bit format (the same bytes, reordered; the page
 * calls such a load-time weight reordering "prepacking"):
 *   Pq uint8 [N, K/2]:   Pq[n, i] = q[2i, n] | q[2i+1, n] << 4  (pairs along K)
 *   Ps fp32  [N, K/32]:  Ps[n, b] = scales[b, n]
 *   Pz uint8 [N, K/64]:  Pz[n, j] = z[2j, n] | z[2j+1, n] << 4  (K % 64 == 0)
 * Status ORC_BAD_SHAPE unless K % 64 == 0 and N even.                      */
int orc_w4_prepack_kmajor(const uint8_t *Wq, const float *scales, const uint8_t *zeros,
                          int64_t K, int64_t N, uint8_t *Pq, float *Ps, uint8_t *Pz);

/* Plain matmul with fp64 accumulation:
 * y[m, n] = fl32(sum_k x[m, k] * W[k, n] + bias[n])  (bias may be NULL),
 * bound[m, n] = 1e-5 * (sum_k |x[m, k] * W[k, n]| + |bias[n]|) + 1e-6,
 * the per-output tolerance a fp32 implementation is held to (bound may be NULL). */
int orc_matmul_f64(const float *x, int64_t M, int64_t K, const float *W, int64_t N,
                   const float *bias, float *y, double *bound);

/* The 4-bit matmul as the page's runtime executes it: dequantize, then matmul. */
int orc_w4_matmul(const float *x, int64_t M, int64_t K,
                  const uint8_t *Wq, const float *scales, const uint8_t *zeros, int64_t N,
                  const float *bias, float *y, double *bound);

/* int8 head quantizer (step 3): per column (token) n of E fp32 [K, N]:
 * hs[n] = max_k |E[k, n]| / 127, Q[k, n] = clamp(rint(E[k, n] / hs[n]), -127, 127),
 * a zero column gives hs = 0 and Q = 0.  Q int8 [K, ldq]; the padding columns
 * N..ldq-1 are written as 0.                                                */
int orc_i8_quantize_head(const float *E, int64_t K, int64_t N, int64_t ldq,
                         int8_t *Q, float *hs);

/* Per-token dequantization of the table: E_hat[k, n] = fl32(Q[k, n] * hs[n]), [K, N]. */
int orc_i8_dequantize_head(const int8_t *Q, int64_t ldq, const float *hs,
                           int64_t K, int64_t N, float *E_hat);

/* Last-token logits (step 4): logits[n] = fl32(sum_k x[k] * E_hat[k, n]) for the
 * one row x [K], accumulated in fp64, with the per-output bound as above.  */
int orc_i8_head_logits(const float *x, int64_t K, const int8_t *Q, int64_t ldq,
                       const float *hs, int64_t N, float *logits, double *bound);

/* Token lookup from the same table (step 3: Gather along axis 1, then
 * Transpose): out[t, k] = E_hat[k, tokens[t]], out fp32 [T, K].
 * A token outside [0, N) is ORC_BAD_SHAPE.                                  */
int orc_i8_embed(const int64_t *tokens, int64_t T, const int8_t *Q, int64_t ldq,
                 const float *hs, int64_t K, int64_t N, float *out);

/* ---- fp16-scale variant of the format (page section "Quantization", the
 * measurements table's "fp16 scales" file): the same codes and zero points,
 * scales stored as IEEE binary16 bit patterns.  Dequantization still gives
 * fp32: W_hat = fl32((q - z) * s) with s the binary16 value, so the fp32
 * functions above apply after orc_f16_array_to_f32 on the scales.          */

/* fp32 -> binary16 bits, round to nearest, ties to even; |f| >= 65520 -> inf. */
uint16_t orc_f32_to_f16(float f);

/* binary16 bits -> fp32 (exact).                                            */
float orc_f16_to_f32(uint16_t h);
void orc_f16_array_to_f32(const uint16_t *h, int64_t count, float *out);

/* Quantizer with binary16 scales: per block s16 = binary16((hi - lo) / 15),
 * then z and q as in orc_w4_quantize_pack against s = s16.  s16 == inf is
 * ORC_NONFINITE; s16 == 0 gives s = z = q = 0.  scales uint16 [K/32, N].    */
int orc_w4h_quantize_pack(const float *W, int64_t K, int64_t N,
                          uint8_t *Wq, uint16_t *scales, uint8_t *zeros);

/* ---- Fused epilogues (pages "rlx-web": a SwiGLU MLP; "zero-tvm": a fused
 * gate + up + SiLU kernel and a fused residual add; GPT-2's MLP activation is
 * GELU, which the pages do not spell out: the tanh form is our reading).
 * t[m, n] = sum_k x[m, k] * W_hat[k, n] + bias[n], kept in fp64, then
 *   ORC_ACT_NONE:   o[m, n] = t[m, n]
 *   ORC_ACT_GELU:   o[m, n] = gelu(t[m, n])
 *   ORC_ACT_SWIGLU: o[m, i] = silu(t[m, 2 i]) * t[m, 2 i + 1]   (N even)
 * (gate and up columns interleaved), y = fl32(o + residual) with residual
 * [M, N_out] optional, N_out = N / 2 for SWIGLU, else N.                   */
enum { ORC_ACT_NONE = 0, ORC_ACT_GELU = 1, ORC_ACT_SWIGLU = 2 };

/* gelu(v) = v / 2 * (1 + tanh(sqrt(2 / pi) * (v + 0.044715 v^3)))          */
double orc_gelu(double v);
/* silu(v) = v / (1 + exp(-v))                                               */
double orc_silu(double v);

/* bound[m, n_out]: the tolerance an fp32 implementation is held to, from the
 * matmul bound B = 1e-5 * (sum_k |x w| + |bias|) + 1e-6 of each pre-activation
 * value carried through the activation's slope (|gelu'| <= 1.13, |silu'| <=
 * 1.1), plus 2^-20 of the magnitudes entering the activation for its fp32
 * evaluation and 2^-23 |y| for the final additions.                        */
int orc_w4_matmul_ep(const float *x, int64_t M, int64_t K,
                     const uint8_t *Wq, const float *scales, const uint8_t *zeros, int64_t N,
                     const float *bias, const float *residual, int act, float *y,
                     double *bound);

/* ---- Group-64 affine variant (zero-tvm README, the kernel A/B table:
 * "4-bit/group-64/affine"; the int4 matmul family it measures).  The page
 * names the format only; this is its plainest reading (R18): per group of
 * 64 consecutive rows k = 64 g .. 64 g + 63 of column n,
 *   lo = min w, hi = max w, s = fl32(fl32(hi - lo) / 15), m = lo,
 *   q = clamp(rint(fl32(fl32(w - lo) / s)), 0, 15)   (s == 0: q = 0),
 *   W_hat = fl32(q * s + m)   (one rounding: fused multiply-add),
 * so the group's minimum is reproduced exactly and the range is the data's
 * own (no zero point).  Codes packed like Wq ([K, N/2], pairs along N, low
 * nibble first); scales and mins fp32 [K/64, N]; 0.625 B/weight.  K % 64 == 0,
 * N even; a non-finite weight or range is ORC_NONFINITE.                    */
#define ORC_GROUP 64
int orc_w4g_quantize_pack(const float *W, int64_t K, int64_t N,
                          uint8_t *Wq, float *scales, float *mins);
int orc_w4g_dequantize(const uint8_t *Wq, const float *scales, const float *mins,
                       int64_t K, int64_t N, float *W_hat);
/* K-major copy: Pq as orc_w4_prepack_kmajor's, Ps and Pm fp32 [N, K/64].     */
int orc_w4g_prepack_kmajor(const uint8_t *Wq, const float *scales, const float *mins,
                           int64_t K, int64_t N, uint8_t *Pq, float *Ps, float *Pm);
/* dequantize, then orc_matmul_f64 (same bound).                             */
int orc_w4g_matmul(const float *x, int64_t M, int64_t K,
                   const uint8_t *Wq, const float *scales, const float *mins, int64_t N,
                   const float *bias, float *y, double *bound);

#ifdef __cplusplus
}
#endif

#endif /* W4_ORACLE_H */
