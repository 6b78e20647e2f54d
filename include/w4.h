/*
 * w4.h -- C ABI of the MI355X (gfx950) 4-bit block-dequant weight matmul and
 * the int8 tied LM head.
 *
 * The method (page "ONNX export, quantization and the browser runtime",
 * section "Quantization (train/quantize.py)"):
 *   step 1  each linear layer of the body is a [K, N] weight matrix and a bias;
 *   step 2  the matrix is kept in 4 bits: in every column, each run of 32
 *           rows is quantized asymmetrically with its own scale (fp32) and
 *           zero point (uint4), codes are packed two to a byte, and
 *           dequantization restores w_hat = (q - z) * scale in fp32;
 *   step 3  the embedding and the LM head share one int8 [768, 50257] table
 *           with an fp32 scale for each token; a token's embedding is its
 *           column of the table;
 *   step 4  logits are needed for the final position alone.
 * The paragraph after the steps: the runtime folds the dequantization and
 * runs fp32 kernels, so every matmul here computes x . w_hat in fp32.
 *
 * Layouts (all row-major, all device memory owned by the caller):
 *   x       fp32  [M, K]
 *   Wq      uint8 [K, N/2]     Wq[k, j] = q[k, 2j] | q[k, 2j+1] << 4
 *   scales  fp32  [K/32, N]    scale of rows 32b..32b+31 of column n
 *   zeros   uint8 [K/32, N/2]  packed like Wq: z[b, 2j] low nibble, z[b, 2j+1] high
 *   bias    fp32  [N]          may be NULL
 *   y       fp32  [M, N]
 *   Q       int8  [K, ldq]     head table, ldq >= N; hs fp32 [N] a scale for each token
 * The pairing of nibbles along N (flat row-major UINT4 packing of the [K, N]
 * code tensor, element 2i in the low nibble) is a reading: the page says
 * only "raw packed UINT4"; low nibble first is fixed.
 *
 * Conventions:
 *   - Return value: W4_OK (0) or a W4_ERR_* code; nothing is thrown.  Every
 *     argument is checked on the host before any HIP call, so a bad call
 *     enqueues nothing.  W4_ERR_LAUNCH carries the HIP error of the launch.
 *   - Sizes are int64_t.  Empty sizes are valid: M == 0 or N == 0 enqueue
 *     nothing; K == 0 makes every output equal to the bias (or 0).
 *   - Pointers are device pointers: 16-byte aligned for Wq, scales, zeros,
 *     the head tables Q and Qt and the activations x of every matmul (read
 *     in 16-byte pieces); 4-byte aligned for the other fp32 arrays (bias, y,
 *     residual, hs, logits).  Each head call states its own rule for x.  A
 *     pointer may be NULL only when the buffer it names is empty, or where
 *     marked "may be NULL".
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Calls only enqueue work on it: they never synchronize, and never
 *     allocate device memory.  Scratch memory is the caller's `workspace`.
 *   - Data-dependent failures that the host cannot see (a non-finite weight)
 *     are reported through the optional device word `d_status`: the kernel
 *     stores W4_ERR_NONFINITE there and leaves it untouched otherwise, so the
 *     caller zeroes it first and reads it after synchronizing.
 *   - All kernels are built for gfx950 only; any other current device gives
 *     W4_ERR_DEVICE.  The library holds no per-call state and is safe to call
 *     from several host threads; two calls that share a workspace must be
 *     ordered on one stream.
 */
#ifndef W4_H
#define W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4_ABI_VERSION 1

enum {
    W4_OK = 0,
    W4_ERR_NULL_PTR = 1,    /* a required pointer is NULL                         */
    W4_ERR_BAD_SHAPE = 2,   /* negative size, K % 32 != 0, N odd, ldq < N, bad token */
    W4_ERR_MISALIGNED = 3,  /* a pointer breaks the alignment rule above          */
    W4_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required            */
    W4_ERR_DEVICE = 5,      /* no current HIP device, or it is not gfx950         */
    W4_ERR_LAUNCH = 6,      /* the kernel launch failed (HIP error)               */
    W4_ERR_NONFINITE = 7    /* device status only: a non-finite input value       */
};

/* Version of this header's ABI (W4_ABI_VERSION). */
int w4_abi_version(void);

/* Static text for a status code; never NULL. */
const char *w4_strerror(int status);

/* ---------------------------------------------------------------------------
 * Block quantizer and packer (step 2).  W fp32 [K, N] -> Wq, scales, zeros.
 * Per block (32 rows of one column): lo = min(0, min w), hi = max(0, max w),
 * s = (hi - lo) / 15 in fp32 with a correctly rounded division; s == 0 gives
 * s = z = q = 0; else z = clamp(rint(-lo / s), 0, 15) and
 * q = clamp(rint(w / s) + z, 0, 15), rint rounding half to even (a reading:
 * ONNX QuantizeLinear's rule; the page states none).  The zero-inclusive
 * range is also a reading: it keeps real 0 representable, so a block whose
 * weights share one sign still meets |w - w_hat| <= s / 2.
 * Output bytes are a deterministic function of W (bit-for-bit reproducible).
 * d_status (may be NULL): set to W4_ERR_NONFINITE if a weight is not finite
 * or a scale overflows; the outputs of such a block are unspecified.
 * ------------------------------------------------------------------------- */
int w4_quantize_pack(const float *W, int64_t K, int64_t N,
                     uint8_t *Wq, float *scales, uint8_t *zeros,
                     int *d_status, void *stream);

/* Unpack codes and zero points one per byte: q uint8 [K, N], z uint8 [K/32, N]. */
int w4_unpack(const uint8_t *Wq, const uint8_t *zeros, int64_t K, int64_t N,
              uint8_t *q, uint8_t *z, void *stream);

/* Blocked dequantization (step 2): W_hat fp32 [K, N],
 * W_hat[k, n] = fl32((q[k, n] - z[k/32, n]) * scales[k/32, n]) -- one fp32
 * multiply of an exact small integer, so the result is bit-exact.          */
int w4_dequantize(const uint8_t *Wq, const float *scales, const uint8_t *zeros,
                  int64_t K, int64_t N, float *W_hat, void *stream);

/* ---------------------------------------------------------------------------
 * 4-bit matmul (steps 1-2 with the folded-fp32 runtime):
 *   y[m, n] = sum_k x[m, k] * w_hat[k, n] + bias[n]
 * computed in fp32 (never TF32 or lower).  Accuracy: every output is within
 * 1e-5 * (sum_k |x[m, k] * w_hat[k, n]| + |bias[n]|) + 1e-6 of the exact
 * value.  M == 1 runs the fused dequant-GEMV; M > 1 runs the dequant-to-LDS
 * fp32-MFMA kernel.  Results are deterministic (no floating-point atomics).
 * bias may be NULL.  Where K is split across workgroups, their partial sums
 * go to the caller's workspace (at least w4_matmul_workspace_bytes(M, K, N)
 * bytes, 256-byte aligned, any contents) and a second kernel on the same
 * stream adds them in a fixed order; a size of 0 means no workspace is used.
 * ------------------------------------------------------------------------- */
size_t w4_matmul_workspace_bytes(int64_t M, int64_t K, int64_t N);

int w4_matmul(const float *x, int64_t M, int64_t K,
              const uint8_t *Wq, const float *scales, const uint8_t *zeros, int64_t N,
              const float *bias, float *y,
              void *workspace, size_t workspace_bytes, void *stream);

/* w4_matmul for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops, harnesses that forbid hipMalloc): the same
 * kernels and result, but split-K partial sums go to a device array that the
 * library holds for the life of the process, W4_NOALLOC_SCRATCH_BYTES bytes
 * on each GPU it runs on.  A shape whose w4_matmul_workspace_bytes exceeds
 * that gives W4_ERR_WORKSPACE (checked on the host, nothing enqueued).  The
 * call allocates nothing.  Every call on one GPU shares that GPU's array,
 * which keeps the last call's contents (the kernels never need it cleared):
 * calls that may overlap on one GPU (different streams, or host threads
 * without ordering) race on it and must be ordered by the caller.  The first
 * call on a device looks up that device's array (a HIP symbol query).    */
#define W4_NOALLOC_SCRATCH_BYTES (32u << 20)

int w4_matmul_noalloc(const float *x, int64_t M, int64_t K,
                      const uint8_t *Wq, const float *scales, const uint8_t *zeros, int64_t N,
                      const float *bias, float *y, void *stream);

/* Argument check of w4_matmul without any HIP call (same return codes,
 * minus W4_ERR_DEVICE / W4_ERR_LAUNCH); usable on a machine with no GPU.   */
int w4_check_matmul_args(const float *x, int64_t M, int64_t K,
                         const uint8_t *Wq, const float *scales, const uint8_t *zeros,
                         int64_t N, const float *bias, const float *y,
                         const void *workspace, size_t workspace_bytes);

/* ---------------------------------------------------------------------------
 * K-major ("prepacked") copy of the same format, for the decode GEMV.  The
 * page mentions the runtime's weight prepacking; here it is a byte-exact
 * reordering that makes each output column's data contiguous:
 *   Pq uint8 [N, K/2]   Pq[n, i] = q[2i, n] | q[2i+1, n] << 4 (pairs along K)
 *   Ps fp32  [N, K/32]  Ps[n, b] = scales[b, n]
 *   Pz uint8 [N, K/64]  Pz[n, j] = z[2j, n] | z[2j+1, n] << 4
 * Same bytes per weight as the canonical layout.  Requires K % 64 == 0.
 * Pq, Ps, Pz are caller-allocated device buffers (16-byte aligned).        */
int w4_prepack_kmajor(const uint8_t *Wq, const float *scales, const uint8_t *zeros,
                      int64_t K, int64_t N, uint8_t *Pq, float *Ps, uint8_t *Pz,
                      void *stream);

/* y = x . w_hat + bias on the K-major layout: same result contract as
 * w4_matmul (fp32, same bound, deterministic).  For M <= 2 (decode), and
 * for any M when K % 128 != 0, every workgroup owns whole columns and no
 * workspace is used.  For M >= 3 with K % 128 == 0 and K < 2^22 (small
 * batches, prefill) the product runs on the matrix cores at fp32 accuracy
 * with exact operands: within a block the scale factors out, (q - z) is
 * exact in bf16, and each activation is split exactly into three bf16
 * terms, so every product is exact and only the fp32 accumulation rounds;
 * the block's scale is applied once per block and column.  This holds for
 * any finite x, whatever its range.  Non-finite x gives NaN outputs on this
 * path.  One workgroup takes 16 or 32 columns of up to 16 rows over all of
 * K (one launch, no workspace) when M <= 16 and N >= 497, and also for
 * 17 to 128 rows, in groups of 16, on matrices of at most 2^22 weights
 * whose column and row groups number at least 32; otherwise it may split K across
 * workgroups and then needs a workspace of
 * w4_matmul_kmajor_workspace_bytes(M, K, N) bytes (0 when it does not):
 * device memory, 256-byte aligned, any contents, not shared with a call in
 * flight on another stream.  Indexing is 32-bit: K * N, M * K and M * N must
 * be below 2^31 (W4_ERR_BAD_SHAPE otherwise).                              */
size_t w4_matmul_kmajor_workspace_bytes(int64_t M, int64_t K, int64_t N);

int w4_matmul_kmajor(const float *x, int64_t M, int64_t K, const uint8_t *Pq, const float *Ps,
                     const uint8_t *Pz, int64_t N, const float *bias, float *y,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Argument check of w4_matmul_kmajor without any HIP call.                 */
int w4_check_matmul_kmajor_args(const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                                const float *Ps, const uint8_t *Pz, int64_t N,
                                const float *bias, const float *y,
                                const void *workspace, size_t workspace_bytes);

/* ---------------------------------------------------------------------------
 * fp16-scale variant (page section "Quantization", the measurements table's
 * "4-bit DequantizeLinear, fp16 scales" file): the same codes and zero points,
 * each block scale stored as an IEEE binary16 bit pattern (uint16), 0.578125
 * bytes per weight.  The quantizer rounds the fp32 scale (hi - lo) / 15 to
 * binary16 (to nearest, ties to even) and takes the zero point and codes
 * against that stored value; a scale that overflows binary16 (>= 65520) sets
 * d_status to W4_ERR_NONFINITE, one that rounds to 0 gives an all-zero block.
 * Dequantization is still fp32: w_hat = fl32((q - z) * s), s the binary16
 * value.  Layouts, alignment, status codes and the result bound are those of
 * the fp32-scale functions of the same name without the h; the K-major
 * matmul needs the workspace w4_matmul_kmajor_workspace_bytes(M, K, N).     */
int w4h_quantize_pack(const float *W, int64_t K, int64_t N, uint8_t *Wq, uint16_t *scales,
                      uint8_t *zeros, int *d_status, void *stream);

int w4h_dequantize(const uint8_t *Wq, const uint16_t *scales, const uint8_t *zeros, int64_t K,
                   int64_t N, float *W_hat, void *stream);

int w4h_prepack_kmajor(const uint8_t *Wq, const uint16_t *scales, const uint8_t *zeros,
                       int64_t K, int64_t N, uint8_t *Pq, uint16_t *Ps, uint8_t *Pz,
                       void *stream);

int w4h_check_matmul_kmajor_args(const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                                 const uint16_t *Ps, const uint8_t *Pz, int64_t N,
                                 const float *bias, const float *y,
                                 const void *workspace, size_t workspace_bytes);

int w4h_matmul_kmajor(const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                      const uint16_t *Ps, const uint8_t *Pz, int64_t N, const float *bias,
                      float *y, void *workspace, size_t workspace_bytes, void *stream);

/* ---- group-64 affine variant ---------------------------------------------
 * The format of zero-tvm's kernel A/B ("4-bit/group-64/affine"; zero-tvm
 * README, the A/B table against LM Studio).  The page names it only; the
 * reading taken: per group of 64 consecutive rows k of column n,
 *   lo = min w, hi = max w, s = (hi - lo) / 15, m = lo        (fp32),
 *   q = clamp(rint((w - lo) / s), 0, 15)  (s = 0: q = 0),
 *   W_hat = fma(q, s, m)                                      (one rounding),
 * so the group minimum is exact and no zero point is stored.
 *   Wq      uint8 [K, N/2]   as in the base format (pairs along N, low first)
 *   scales  fp32  [K/64, N]
 *   mins    fp32  [K/64, N]
 * 0.625 B/weight.  K % 64 == 0, N even; arrays 16-byte aligned.  Quantize,
 * dequantize and the K-major copy are bit-exact; a non-finite weight or range
 * sets *d_status = W4_ERR_NONFINITE (as w4_quantize_pack).                 */
int w4g_quantize_pack(const float *W, int64_t K, int64_t N, uint8_t *Wq, float *scales,
                      float *mins, int *d_status, void *stream);

int w4g_dequantize(const uint8_t *Wq, const float *scales, const float *mins, int64_t K,
                   int64_t N, float *W_hat, void *stream);

/* K-major copy: Pq uint8 [N, K/2] (as w4_prepack_kmajor), Ps and Pm fp32
 * [N, K/64] (scales and minima transposed).                                */
int w4g_prepack_kmajor(const uint8_t *Wq, const float *scales, const float *mins, int64_t K,
                       int64_t N, uint8_t *Pq, float *Ps, float *Pm, void *stream);

/* y [M, N] = x [M, K] . W_hat (+ bias), on the K-major copy; every output
 * within the bound of w4_matmul.  The decode GEMV for every M (rows four at a
 * time; M <= 262140); no workspace, one launch.                            */
int w4g_check_matmul_kmajor_args(const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                                 const float *Ps, const float *Pm, int64_t N, const float *bias,
                                 const float *y);

int w4g_matmul_kmajor(const float *x, int64_t M, int64_t K, const uint8_t *Pq, const float *Ps,
                      const float *Pm, int64_t N, const float *bias, float *y, void *stream);

/* ---- fused epilogues on the K-major matmul -------------------------------
 * Pages "rlx-web" (a SwiGLU MLP) and "zero-tvm" (a fused gate + up + SiLU
 * kernel, a fused residual add); GPT-2's MLP activation, GELU, in its tanh
 * form.  With t = x . W_hat + bias as w4_matmul_kmajor computes it:
 *   W4_ACT_NONE    y[m, n] = t[m, n]                              [M, N]
 *   W4_ACT_GELU    y[m, n] = gelu(t[m, n]),
 *                  gelu(v) = v/2 (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))
 *   W4_ACT_SWIGLU  y[m, i] = silu(t[m, 2i]) * t[m, 2i+1],  silu(v) = v / (1 + e^-v)
 *                  (gate and up columns interleaved by the caller; y is [M, N/2])
 * then y += residual (fp32, same shape as y, 4-byte aligned; may be y itself
 * for an in-place residual add, no other overlap).  Every output is within
 * the matmul bound carried through the activation's slope (|gelu'| <= 1.13,
 * |silu'| <= 1.1) plus a few fp32 roundings of the activation's evaluation.
 * Workspace: w4_matmul_kmajor_workspace_bytes(M, K, N).  An unknown act is
 * W4_ERR_BAD_SHAPE.                                                        */
#define W4_ACT_NONE 0
#define W4_ACT_GELU 1
#define W4_ACT_SWIGLU 2

int w4_check_matmul_kmajor_ep_args(const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                                   const float *Ps, const uint8_t *Pz, int64_t N,
                                   const float *bias, const float *residual, int act,
                                   const float *y, const void *workspace,
                                   size_t workspace_bytes);

int w4_matmul_kmajor_ep(const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                        const float *Ps, const uint8_t *Pz, int64_t N, const float *bias,
                        const float *residual, int act, float *y, void *workspace,
                        size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * int8 tied head (step 3).  E fp32 [K, N] -> Q int8 [K, ldq], hs fp32 [N]:
 * hs[n] = max_k |E[k, n]| / 127 (correctly rounded fp32 division),
 * Q[k, n] = clamp(rint(E[k, n] / hs[n]), -127, 127); a zero column gives
 * hs = 0 and Q = 0; padding columns N..ldq-1 are written as 0.  Bit-exact.
 * d_status (may be NULL) reports a non-finite entry.                       */
int i8_quantize_head(const float *E, int64_t K, int64_t N, int64_t ldq,
                     int8_t *Q, float *hs, int *d_status, void *stream);

/* Last-token logits (step 4): logits[n] = sum_k x_last[k] * fl32(Q[k, n] * hs[n]),
 * fp32, within the same bound as w4_matmul.  x_last is the last row of the
 * activations (the caller passes x + (M - 1) * K).  Any ldq >= N works;
 * ldq % 16 == 0 takes the 16-byte-load path.  The workspace rule is that of
 * w4_matmul, with size i8_head_workspace_bytes(K, N).                      */
size_t i8_head_workspace_bytes(int64_t K, int64_t N);

int i8_head_logits(const float *x_last, int64_t K, const int8_t *Q, int64_t ldq,
                   const float *hs, int64_t N, float *logits,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Token lookup from the same table (step 3: gather along axis 1, then
 * transpose): out[t, k] = fl32(Q[k, tokens[t]] * hs[tokens[t]]), fp32 [T, K],
 * bit-exact.  tokens int64 [T] on the device; an id outside [0, N) sets
 * d_status (may be NULL) to W4_ERR_BAD_SHAPE and yields a zero row.        */
int i8_embed(const int64_t *tokens, int64_t T, const int8_t *Q, int64_t ldq,
             const float *hs, int64_t K, int64_t N, float *out,
             int *d_status, void *stream);

/* ---- int8 head on a K-major copy of the table -------------------------------
 * Same method (steps 3-4), table stored token-major: Qt int8 [N, ldt] with
 * Qt[n, k] = Q[k, n], each row zero-padded to ldt >= K, ldt % 16 == 0, and
 * N * ldt < 2^31.  Row n is token n's embedding vector, contiguous.        */

/* Byte-exact relayout of Q [K, ldq] into Qt [N, ldt] (columns K..ldt-1 of Qt
 * set to 0).  Q and Qt are 16-byte aligned.                                 */
int i8_prepack_head(const int8_t *Q, int64_t K, int64_t N, int64_t ldq,
                    int8_t *Qt, int64_t ldt, void *stream);

/* Host-only validation of i8_head_logits_kmajor's arguments.               */
int i8_check_head_logits_kmajor_args(const float *x_last, int64_t K, const int8_t *Qt,
                                     int64_t ldt, const float *hs, int64_t N,
                                     const float *logits);

/* Last-token logits: logits[n] = hs[n] * sum_k x_last[k] * Qt[n, k], one
 * launch, no workspace.  K % 16 == 0, 16 <= K <= 8192.  fp32 arithmetic with
 * every product formed exactly from the int8 code and the fp32 activation, so
 * every logit is within the bound of w4_matmul for any finite x_last (nothing
 * of x is quantized).  A non-finite entry of x_last gives NaN logits.
 * x_last, Qt 16-byte aligned; hs, logits 4-byte aligned.                   */
int i8_head_logits_kmajor(const float *x_last, int64_t K, const int8_t *Qt, int64_t ldt,
                          const float *hs, int64_t N, float *logits, void *stream);

/* Full-sequence logits (the page's export before the last-position slice of
 * step 4): logits[m, n] = hs[n] * sum_k x[m, k] * Qt[n, k] for every row m of
 * x [M, K] (fp32, row-major, 16-byte aligned), logits [M, N] fp32.  Every
 * product is exact and only fp32 accumulation rounds (from 4 rows with K <=
 * 1024 on the bf16 matrix cores, each activation split exactly into three
 * bf16 parts; otherwise as i8_head_logits_kmajor), so the bound is that of
 * i8_head_logits_kmajor (a row with a non-finite entry gives NaN logits for
 * that row only).  K % 16 == 0, 16 <= K <= 8192;
 * N * ldt < 2^31.  One launch; no workspace is needed:
 * i8_head_rows_workspace_bytes returns 0 and `workspace` may be NULL.      */
size_t i8_head_rows_workspace_bytes(int64_t M, int64_t K);

int i8_check_head_logits_rows_args(const float *x, int64_t M, int64_t K, const int8_t *Qt,
                                   int64_t ldt, const float *hs, int64_t N,
                                   const float *logits, const void *workspace,
                                   size_t workspace_bytes);

int i8_head_logits_rows(const float *x, int64_t M, int64_t K, const int8_t *Qt, int64_t ldt,
                        const float *hs, int64_t N, float *logits, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Token lookup from Qt (step 3): out[t, k] = fl32(Qt[tokens[t], k] * hs[tokens[t]]),
 * fp32 [T, K], bit-exact; ids outside [0, N) as in i8_embed.               */
int i8_embed_kmajor(const int64_t *tokens, int64_t T, const int8_t *Qt, int64_t ldt,
                    const float *hs, int64_t K, int64_t N, float *out,
                    int *d_status, void *stream);

/* ---- measurement: streaming-read reference ---------------------------------
 * Reads [src, src + bytes) once with 16-byte streaming loads, loads_per_lane
 * (4, 6, 8, 12 or 16) of them per lane, 256 lanes (4 waves) per workgroup,
 * and writes out[w] = XOR of the 32-bit words wave w read, for w below
 * w4_read_bytes_words(bytes, loads_per_lane) (0 for arguments out of range):
 * lane t of workgroup g reads the 16-byte pieces g 256 + t + j 256 G (G
 * workgroups, j < loads_per_lane) that lie below bytes.
 * The benchmark times one launch per weight matrix, each over that matrix's
 * packed byte count, as the launch floor of the decode pass: the same bytes
 * and launches as the GEMV, without its arithmetic.  bytes % 16 == 0; src
 * 16-byte aligned, out 4-byte aligned.                                      */
size_t w4_read_bytes_words(int64_t bytes, int loads_per_lane);

int w4_read_bytes(const void *src, int64_t bytes, int loads_per_lane, uint32_t *out,
                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W4_H */
