/*
 * CPU oracle: plain, slow, obviously correct.  TEST INFRASTRUCTURE ONLY (see
 * oracle.h).  Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off
 * -fopenmp.  No intrinsics, no blocking: every output is one loop over its
 * definition.  The matmul and the dequantization share their independent
 * outputs (columns, rows) among OpenMP threads; each output's own loop runs
 * in order, so the results do not depend on the thread count.  fp32 steps are
 * written as fp32 expressions (x86-64 evaluates float in float); fp64 steps
 * are explicit casts to double.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BLOCK 32

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int bad_w4_shape(int64_t K, int64_t N)
{
    return K < 0 || N < 0 || K % BLOCK != 0 || N % 2 != 0;
}

void orc_pack_u4(const uint8_t *v, int64_t count, uint8_t *out)
{
    for (int64_t i = 0; i < count / 2; ++i)
        out[i] = (uint8_t)((v[2 * i] & 15) | ((v[2 * i + 1] & 15) << 4));
}

void orc_unpack_u4(const uint8_t *in, int64_t count, uint8_t *v)
{
    for (int64_t i = 0; i < count / 2; ++i) {
        v[2 * i] = (uint8_t)(in[i] & 15);
        v[2 * i + 1] = (uint8_t)(in[i] >> 4);
    }
}

/* clamp a float that holds an integer value into [lo, hi] and return it as int */
static int clamp_int(float v, int lo, int hi)
{
    if (v < (float)lo) return lo;
    if (v > (float)hi) return hi;
    return (int)v;
}

/* One block: 32 weights w[r * stride], r = 0..31.  Writes s, z and q[0..31].
 * With s16_out != NULL the scale is stored as binary16 (the fp16-scale
 * variant): s16 = binary16((hi - lo) / 15) goes to *s16_out and z, q are taken
 * against its value; s16 infinite is ORC_NONFINITE, s16 == 0 gives zeros.   */
static int quantize_block(const float *w, int64_t stride, float *s_out, uint16_t *s16_out,
                          uint8_t *z_out, uint8_t *q_out)
{
    float lo = 0.0f, hi = 0.0f; /* the range always contains 0 */
    for (int r = 0; r < BLOCK; ++r) {
        float v = w[r * stride];
        if (!isfinite(v)) return ORC_NONFINITE;
        if (v < lo) lo = v;
        if (v > hi) hi = v;
    }
    float range = hi - lo;
    float s = range / 15.0f;
    if (!isfinite(s)) return ORC_NONFINITE;
    if (s16_out) {
        uint16_t h = orc_f32_to_f16(s);
        if ((h & 0x7C00) == 0x7C00) return ORC_NONFINITE;
        *s16_out = h;
        s = orc_f16_to_f32(h); /* the stored value */
    }
    if (s == 0.0f) { /* all-zero block: every code and the zero point are 0 */
        if (s_out) *s_out = 0.0f;
        *z_out = 0;
        for (int r = 0; r < BLOCK; ++r) q_out[r] = 0;
        return ORC_OK;
    }
    float zr = rintf(-lo / s);
    int z = clamp_int(zr, 0, 15);
    for (int r = 0; r < BLOCK; ++r) {
        float t = rintf(w[r * stride] / s);
        q_out[r] = (uint8_t)clamp_int(t + (float)z, 0, 15);
    }
    if (s_out) *s_out = s;
    *z_out = (uint8_t)z;
    return ORC_OK;
}

int orc_w4_quantize_pack(const float *W, int64_t K, int64_t N,
                         uint8_t *Wq, float *scales, uint8_t *zeros)
{
    if (bad_w4_shape(K, N)) return ORC_BAD_SHAPE;
    int64_t nb = K / BLOCK;
    uint8_t *q = (uint8_t *)malloc((size_t)(K * N) + 1);
    uint8_t *z = (uint8_t *)malloc((size_t)(nb * N) + 1);
    if (!q || !z) { free(q); free(z); return ORC_NO_MEMORY; }
    int st = ORC_OK;
    uint8_t qcol[BLOCK];
    for (int64_t b = 0; b < nb && st == ORC_OK; ++b) {
        for (int64_t n = 0; n < N; ++n) {
            st = quantize_block(W + (b * BLOCK) * N + n, N, &scales[b * N + n], NULL,
                                &z[b * N + n], qcol);
            if (st != ORC_OK) break;
            for (int r = 0; r < BLOCK; ++r) q[(b * BLOCK + r) * N + n] = qcol[r];
        }
    }
    if (st == ORC_OK) {
        orc_pack_u4(q, K * N, Wq);
        orc_pack_u4(z, nb * N, zeros);
    }
    free(q);
    free(z);
    return st;
}

int orc_w4_unpack(const uint8_t *Wq, const uint8_t *zeros, int64_t K, int64_t N,
                  uint8_t *q, uint8_t *z)
{
    if (bad_w4_shape(K, N)) return ORC_BAD_SHAPE;
    orc_unpack_u4(Wq, K * N, q);
    orc_unpack_u4(zeros, (K / BLOCK) * N, z);
    return ORC_OK;
}

int orc_w4_dequantize(const uint8_t *Wq, const float *scales, const uint8_t *zeros,
                      int64_t K, int64_t N, float *W_hat)
{
    if (bad_w4_shape(K, N)) return ORC_BAD_SHAPE;
    uint8_t *q = (uint8_t *)malloc((size_t)(K * N) + 1);
    uint8_t *z = (uint8_t *)malloc((size_t)((K / BLOCK) * N) + 1);
    if (!q || !z) { free(q); free(z); return ORC_NO_MEMORY; }
    orc_w4_unpack(Wq, zeros, K, N, q, z);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t blk = (k / BLOCK) * N + n;
            int diff = (int)q[k * N + n] - (int)z[blk];
            /* the fp64 product of a small integer and a float is exact; the
             * cast is the single fp32 rounding of the dequantized value */
            W_hat[k * N + n] = (float)((double)diff * (double)scales[blk]);
        }
    }
    free(q);
    free(z);
    return ORC_OK;
}

/* Codes of the [K, N] tensor packed along N -> column-major, packed along K.  */
static int transpose_codes(const uint8_t *Wq, int64_t K, int64_t N, uint8_t *Pq)
{
    uint8_t *q = (uint8_t *)malloc((size_t)(K * N) + 1);
    uint8_t *qt = (uint8_t *)malloc((size_t)(K * N) + 1);
    if (!q || !qt) { free(q); free(qt); return ORC_NO_MEMORY; }
    orc_unpack_u4(Wq, K * N, q);
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) qt[n * K + k] = q[k * N + n];
    orc_pack_u4(qt, K * N, Pq);
    free(q);
    free(qt);
    return ORC_OK;
}

int orc_w4_prepack_kmajor(const uint8_t *Wq, const float *scales, const uint8_t *zeros,
                          int64_t K, int64_t N, uint8_t *Pq, float *Ps, uint8_t *Pz)
{
    if (bad_w4_shape(K, N) || K % 64 != 0) return ORC_BAD_SHAPE;
    int64_t nb = K / BLOCK;
    uint8_t *z = (uint8_t *)malloc((size_t)(nb * N) + 1);
    uint8_t *zt = (uint8_t *)malloc((size_t)(nb * N) + 1);
    if (!z || !zt) { free(z); free(zt); return ORC_NO_MEMORY; }
    int st = transpose_codes(Wq, K, N, Pq);
    /* the zero points and scales go column-major the same way */
    orc_unpack_u4(zeros, nb * N, z);
    for (int64_t b = 0; b < nb; ++b)
        for (int64_t n = 0; n < N; ++n) {
            zt[n * nb + b] = z[b * N + n];
            Ps[n * nb + b] = scales[b * N + n];
        }
    orc_pack_u4(zt, nb * N, Pz);
    free(z); free(zt);
    return st;
}

/* Row m of x . W + bias in fp64 (t[n], unrounded) and each output's bound
 * 1e-5 * (sum_k |x w| + |bias|) + 1e-6 (tb[n]).                             */
static void row_f64(const float *xr, int64_t K, const float *W, int64_t N, const float *bias,
                    double *t, double *tb)
{
    /* output columns are independent and each one's sum runs over k in order,
     * so the result does not depend on how many threads share the columns */
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = (double)xr[k] * (double)W[k * N + n];
            acc += p;
            mag += fabs(p);
        }
        if (bias) {
            acc += (double)bias[n];
            mag += fabs((double)bias[n]);
        }
        t[n] = acc;
        tb[n] = 1e-5 * mag + 1e-6;
    }
}

int orc_matmul_f64(const float *x, int64_t M, int64_t K, const float *W, int64_t N,
                   const float *bias, float *y, double *bound)
{
    if (M < 0 || K < 0 || N < 0) return ORC_BAD_SHAPE;
    double *t = (double *)malloc((size_t)N * sizeof(double) + 1);
    double *tb = (double *)malloc((size_t)N * sizeof(double) + 1);
    if (!t || !tb) {
        free(t);
        free(tb);
        return ORC_NO_MEMORY;
    }
    for (int64_t m = 0; m < M; ++m) {
        row_f64(x + m * K, K, W, N, bias, t, tb);
        for (int64_t n = 0; n < N; ++n) {
            y[m * N + n] = (float)t[n];
            if (bound) bound[m * N + n] = tb[n];
        }
    }
    free(t);
    free(tb);
    return ORC_OK;
}

int orc_w4_matmul(const float *x, int64_t M, int64_t K,
                  const uint8_t *Wq, const float *scales, const uint8_t *zeros, int64_t N,
                  const float *bias, float *y, double *bound)
{
    if (M < 0 || bad_w4_shape(K, N)) return ORC_BAD_SHAPE;
    float *W_hat = (float *)malloc((size_t)(K * N) * sizeof(float) + 1);
    if (!W_hat) return ORC_NO_MEMORY;
    int st = orc_w4_dequantize(Wq, scales, zeros, K, N, W_hat);
    if (st == ORC_OK) st = orc_matmul_f64(x, M, K, W_hat, N, bias, y, bound);
    free(W_hat);
    return st;
}

int orc_i8_quantize_head(const float *E, int64_t K, int64_t N, int64_t ldq,
                         int8_t *Q, float *hs)
{
    if (K < 0 || N < 0 || ldq < N) return ORC_BAD_SHAPE;
    for (int64_t n = 0; n < N; ++n) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = E[k * N + n];
            if (!isfinite(v)) return ORC_NONFINITE;
            if (fabsf(v) > amax) amax = fabsf(v);
        }
        float s = amax / 127.0f;
        hs[n] = s;
        for (int64_t k = 0; k < K; ++k) {
            int qv = 0;
            if (s != 0.0f) qv = clamp_int(rintf(E[k * N + n] / s), -127, 127);
            Q[k * ldq + n] = (int8_t)qv;
        }
    }
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = N; n < ldq; ++n) Q[k * ldq + n] = 0;
    return ORC_OK;
}

int orc_i8_dequantize_head(const int8_t *Q, int64_t ldq, const float *hs,
                           int64_t K, int64_t N, float *E_hat)
{
    if (K < 0 || N < 0 || ldq < N) return ORC_BAD_SHAPE;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            E_hat[k * N + n] = (float)((double)Q[k * ldq + n] * (double)hs[n]);
    return ORC_OK;
}

int orc_i8_head_logits(const float *x, int64_t K, const int8_t *Q, int64_t ldq,
                       const float *hs, int64_t N, float *logits, double *bound)
{
    if (K < 0 || N < 0 || ldq < N) return ORC_BAD_SHAPE;
    float *E_hat = (float *)malloc((size_t)(K * N) * sizeof(float) + 1);
    if (!E_hat) return ORC_NO_MEMORY;
    orc_i8_dequantize_head(Q, ldq, hs, K, N, E_hat);
    int st = orc_matmul_f64(x, 1, K, E_hat, N, NULL, logits, bound);
    free(E_hat);
    return st;
}

int orc_i8_embed(const int64_t *tokens, int64_t T, const int8_t *Q, int64_t ldq,
                 const float *hs, int64_t K, int64_t N, float *out)
{
    if (T < 0 || K < 0 || N < 0 || ldq < N) return ORC_BAD_SHAPE;
    for (int64_t t = 0; t < T; ++t)
        if (tokens[t] < 0 || tokens[t] >= N) return ORC_BAD_SHAPE;
    for (int64_t t = 0; t < T; ++t) {
        int64_t tok = tokens[t];
        for (int64_t k = 0; k < K; ++k)
            out[t * K + k] = (float)((double)Q[k * ldq + tok] * (double)hs[tok]);
    }
    return ORC_OK;
}

/* ---- fp16-scale variant ------------------------------------------------------ */

/* fp32 -> IEEE binary16 (1 sign bit, 5 exponent bits with bias 15, 10 fraction
 * bits), rounded to nearest with ties to even.  Straight from the format: the
 * representable values near |f| are the multiples of a quantum, 2^(e-10) for
 * a normal value with exponent e in [-14, 15] and 2^-24 below 2^-14, so |f| is
 * rounded to a multiple of its quantum with rint (ties to even), in double,
 * where the division by a power of two and rint are exact.  |f| >= 65520 (the
 * midpoint above 65504, rounding to even = upward) becomes infinity.        */
uint16_t orc_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f)) return (uint16_t)(sign | 0x7E00);
    double a = fabs((double)f);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e); /* a = m 2^e, m in [0.5, 1): the binary exponent of a is e - 1 */
    int be = e - 1;
    if (be < -14) be = -14; /* subnormal range: quantum 2^-24 */
    double quantum = ldexp(1.0, be - 10);
    double units = rint(a / quantum); /* in [0, 2048] */
    double v = units * quantum;       /* the rounded magnitude */
    if (v == 0.0) return sign;
    if (v < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)units); /* subnormal */
    frexp(v, &e);
    int ev = e - 1; /* exponent of the rounded value (may be be + 1) */
    double frac = v / ldexp(1.0, ev) - 1.0; /* in [0, 1), a multiple of 2^-10 */
    return (uint16_t)(sign | (uint16_t)((ev + 15) << 10) | (uint16_t)(frac * 1024.0));
}

/* IEEE binary16 -> fp32 (exact: every binary16 value is an fp32 value).      */
float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1, ex = (h >> 10) & 31, fr = h & 1023;
    double v;
    if (ex == 0) v = ldexp((double)fr, -24);
    else if (ex == 31) v = fr ? NAN : INFINITY;
    else v = ldexp(1.0 + fr / 1024.0, ex - 15);
    return (float)(sign ? -v : v);
}

int orc_w4h_quantize_pack(const float *W, int64_t K, int64_t N,
                          uint8_t *Wq, uint16_t *scales, uint8_t *zeros)
{
    if (bad_w4_shape(K, N)) return ORC_BAD_SHAPE;
    int64_t nb = K / BLOCK;
    uint8_t *q = (uint8_t *)malloc((size_t)(K * N) + 1);
    uint8_t *z = (uint8_t *)malloc((size_t)(nb * N) + 1);
    if (!q || !z) { free(q); free(z); return ORC_NO_MEMORY; }
    int st = ORC_OK;
    uint8_t qcol[BLOCK];
    for (int64_t b = 0; b < nb && st == ORC_OK; ++b) {
        for (int64_t n = 0; n < N; ++n) {
            st = quantize_block(W + (b * BLOCK) * N + n, N, NULL, &scales[b * N + n],
                                &z[b * N + n], qcol);
            if (st != ORC_OK) break;
            for (int r = 0; r < BLOCK; ++r) q[(b * BLOCK + r) * N + n] = qcol[r];
        }
    }
    if (st == ORC_OK) {
        orc_pack_u4(q, K * N, Wq);
        orc_pack_u4(z, nb * N, zeros);
    }
    free(q);
    free(z);
    return st;
}

void orc_f16_array_to_f32(const uint16_t *h, int64_t count, float *out)
{
    for (int64_t i = 0; i < count; ++i) out[i] = orc_f16_to_f32(h[i]);
}

/* ---- fused epilogues ---------------------------------------------------- */

double orc_gelu(double v)
{
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * v * (1.0 + tanh(c * (v + 0.044715 * v * v * v)));
}

double orc_silu(double v)
{
    return v / (1.0 + exp(-v));
}

int orc_w4_matmul_ep(const float *x, int64_t M, int64_t K,
                     const uint8_t *Wq, const float *scales, const uint8_t *zeros, int64_t N,
                     const float *bias, const float *residual, int act, float *y,
                     double *bound)
{
    if (M < 0 || bad_w4_shape(K, N)) return ORC_BAD_SHAPE;
    if (act != ORC_ACT_NONE && act != ORC_ACT_GELU && act != ORC_ACT_SWIGLU)
        return ORC_BAD_SHAPE;
    if (act == ORC_ACT_SWIGLU && N % 2 != 0) return ORC_BAD_SHAPE;
    const int64_t nout = act == ORC_ACT_SWIGLU ? N / 2 : N;
    float *W_hat = (float *)malloc((size_t)(K * N) * sizeof(float) + 1);
    double *t = (double *)malloc((size_t)N * sizeof(double) + 1);
    double *tb = (double *)malloc((size_t)N * sizeof(double) + 1);
    if (!W_hat || !t || !tb) {
        free(W_hat);
        free(t);
        free(tb);
        return ORC_NO_MEMORY;
    }
    int st = orc_w4_dequantize(Wq, scales, zeros, K, N, W_hat);
    for (int64_t m = 0; st == ORC_OK && m < M; ++m) {
        row_f64(x + m * K, K, W_hat, N, bias, t, tb);  /* pre-activation values */
        for (int64_t i = 0; i < nout; ++i) {
            double o, b;
            if (act == ORC_ACT_SWIGLU) {
                const double g = t[2 * i], u = t[2 * i + 1], sg = orc_silu(g);
                o = sg * u;
                b = 1.1 * fabs(u) * tb[2 * i] + fabs(sg) * tb[2 * i + 1] +
                    ldexp(fabs(g) * fabs(u) + fabs(o), -20);
            } else if (act == ORC_ACT_GELU) {
                o = orc_gelu(t[i]);
                b = 1.13 * tb[i] + ldexp(fabs(t[i]) + fabs(o), -20);
            } else {
                o = t[i];
                b = tb[i];
            }
            if (residual) o += (double)residual[m * nout + i];
            y[m * nout + i] = (float)o;
            if (bound) bound[m * nout + i] = b + ldexp(fabs(o), -23);
        }
    }
    free(W_hat);
    free(t);
    free(tb);
    return st;
}

/* ---- group-64 affine variant -------------------------------------------- */

static int bad_w4g_shape(int64_t K, int64_t N)
{
    return K < 0 || N < 0 || K % ORC_GROUP != 0 || N % 2 != 0;
}

int orc_w4g_quantize_pack(const float *W, int64_t K, int64_t N,
                          uint8_t *Wq, float *scales, float *mins)
{
    if (bad_w4g_shape(K, N)) return ORC_BAD_SHAPE;
    uint8_t *q = (uint8_t *)malloc((size_t)(K * N) + 1);
    if (!q) return ORC_NO_MEMORY;
    int st = ORC_OK;
    for (int64_t g = 0; g < K / ORC_GROUP && st == ORC_OK; ++g) {
        for (int64_t n = 0; n < N && st == ORC_OK; ++n) {
            const float *w = W + (g * ORC_GROUP) * N + n;
            float lo = w[0], hi = w[0];
            for (int r = 0; r < ORC_GROUP; ++r) {
                float v = w[r * N];
                if (!isfinite(v)) { st = ORC_NONFINITE; break; }
                if (v < lo) lo = v;
                if (v > hi) hi = v;
            }
            if (st != ORC_OK) break;
            float range = hi - lo;
            float sc = range / 15.0f;
            if (!isfinite(sc)) { st = ORC_NONFINITE; break; }
            scales[g * N + n] = sc;
            mins[g * N + n] = lo;
            for (int r = 0; r < ORC_GROUP; ++r) {
                int qv = 0;
                if (sc != 0.0f) {
                    float d = w[r * N] - lo;
                    qv = clamp_int(rintf(d / sc), 0, 15);
                }
                q[(g * ORC_GROUP + r) * N + n] = (uint8_t)qv;
            }
        }
    }
    if (st == ORC_OK) orc_pack_u4(q, K * N, Wq);
    free(q);
    return st;
}

int orc_w4g_dequantize(const uint8_t *Wq, const float *scales, const float *mins,
                       int64_t K, int64_t N, float *W_hat)
{
    if (bad_w4g_shape(K, N)) return ORC_BAD_SHAPE;
    uint8_t *q = (uint8_t *)malloc((size_t)(K * N) + 1);
    if (!q) return ORC_NO_MEMORY;
    orc_unpack_u4(Wq, K * N, q);
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            int64_t grp = (k / ORC_GROUP) * N + n;
            /* C99 fmaf: q * s + m with a single rounding */
            W_hat[k * N + n] = fmaf((float)q[k * N + n], scales[grp], mins[grp]);
        }
    free(q);
    return ORC_OK;
}

int orc_w4g_prepack_kmajor(const uint8_t *Wq, const float *scales, const float *mins,
                           int64_t K, int64_t N, uint8_t *Pq, float *Ps, float *Pm)
{
    if (bad_w4g_shape(K, N)) return ORC_BAD_SHAPE;
    int st = transpose_codes(Wq, K, N, Pq);
    const int64_t ng = K / ORC_GROUP;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < ng; ++g) {
            Ps[n * ng + g] = scales[g * N + n];
            Pm[n * ng + g] = mins[g * N + n];
        }
    return st;
}

int orc_w4g_matmul(const float *x, int64_t M, int64_t K,
                   const uint8_t *Wq, const float *scales, const float *mins, int64_t N,
                   const float *bias, float *y, double *bound)
{
    if (M < 0 || bad_w4g_shape(K, N)) return ORC_BAD_SHAPE;
    float *W_hat = (float *)malloc((size_t)(K * N) * sizeof(float) + 1);
    if (!W_hat) return ORC_NO_MEMORY;
    int st = orc_w4g_dequantize(Wq, scales, mins, K, N, W_hat);
    if (st == ORC_OK) st = orc_matmul_f64(x, M, K, W_hat, N, bias, y, bound);
    free(W_hat);
    return st;
}
