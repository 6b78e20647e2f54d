/*
 * Calls every function of the CPU oracle on small inputs, for a build under
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py).
 * Exit status 0 when every call returns the status it should; a sanitizer
 * report ends the process with a nonzero status of its own.  Test
 * infrastructure only: nothing here runs on a GPU.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static int failures = 0;

#define EXPECT(cond)                                                       \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,   \
                    __LINE__, #cond);                                      \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

/* a small deterministic generator (not the method's arithmetic) */
static uint32_t rng_state = 12345u;
static float rnd(void)
{
    rng_state = rng_state * 1664525u + 1013904223u;
    return (float)((int32_t)(rng_state >> 8) - (1 << 23)) / (float)(1 << 23);
}

static void *xmalloc(size_t n) { void *p = malloc(n ? n : 1); if (!p) exit(3); return p; }

int main(void)
{
    enum { K = 96, N = 10, M = 3, KG = 128, V = 37, T = 5 };
    float *W = xmalloc(sizeof(float) * K * N), *x = xmalloc(sizeof(float) * M * KG);
    float *bias = xmalloc(sizeof(float) * N), *res = xmalloc(sizeof(float) * M * N);
    for (int i = 0; i < K * N; ++i) W[i] = 0.02f * rnd();
    for (int i = 0; i < M * KG; ++i) x[i] = rnd();
    for (int i = 0; i < N; ++i) bias[i] = 0.02f * rnd();
    for (int i = 0; i < M * N; ++i) res[i] = rnd();
    for (int k = 0; k < 32; ++k) { W[k * N + 0] = 0.0f; W[k * N + 1] = 0.5f; }  /* degenerate blocks */

    /* packing */
    uint8_t v[16], pk[8], back[16];
    for (int i = 0; i < 16; ++i) v[i] = (uint8_t)i;
    orc_pack_u4(v, 16, pk);
    orc_unpack_u4(pk, 16, back);
    EXPECT(memcmp(v, back, 16) == 0);

    /* the base format */
    uint8_t *Wq = xmalloc(K * N / 2), *zeros = xmalloc(K / 32 * N / 2);
    float *scales = xmalloc(sizeof(float) * K / 32 * N), *What = xmalloc(sizeof(float) * K * N);
    uint8_t *q = xmalloc(K * N), *z = xmalloc(K / 32 * N);
    EXPECT(orc_w4_quantize_pack(W, K, N, Wq, scales, zeros) == ORC_OK);
    EXPECT(orc_w4_unpack(Wq, zeros, K, N, q, z) == ORC_OK);
    EXPECT(orc_w4_dequantize(Wq, scales, zeros, K, N, What) == ORC_OK);
    EXPECT(orc_w4_quantize_pack(W, K + 1, N, Wq, scales, zeros) == ORC_BAD_SHAPE);
    uint8_t *Pq = xmalloc(K * N / 2), *Pz = xmalloc(K / 64 * N + 1);
    float *Ps = xmalloc(sizeof(float) * K / 32 * N);
    EXPECT(orc_w4_prepack_kmajor(Wq, scales, zeros, 64, N, Pq, Ps, Pz) == ORC_OK);
    float *y = xmalloc(sizeof(float) * M * N);
    double *bound = xmalloc(sizeof(double) * M * N);
    EXPECT(orc_matmul_f64(x, M, K, What, N, bias, y, bound) == ORC_OK);
    EXPECT(orc_w4_matmul(x, M, K, Wq, scales, zeros, N, bias, y, bound) == ORC_OK);
    EXPECT(orc_w4_matmul(x, 0, K, Wq, scales, zeros, N, NULL, y, NULL) == ORC_OK);
    W[5] = NAN;
    EXPECT(orc_w4_quantize_pack(W, K, N, Wq, scales, zeros) == ORC_NONFINITE);
    W[5] = 0.01f;

    /* fp16 scales */
    uint16_t *s16 = xmalloc(sizeof(uint16_t) * K / 32 * N);
    float *s16f = xmalloc(sizeof(float) * K / 32 * N);
    EXPECT(orc_w4h_quantize_pack(W, K, N, Wq, s16, zeros) == ORC_OK);
    orc_f16_array_to_f32(s16, K / 32 * N, s16f);
    EXPECT(orc_f16_to_f32(orc_f32_to_f16(0.5f)) == 0.5f);

    /* fused epilogues */
    EXPECT(orc_w4_quantize_pack(W, K, N, Wq, scales, zeros) == ORC_OK);
    for (int act = 0; act <= 2; ++act)
        EXPECT(orc_w4_matmul_ep(x, M, K, Wq, scales, zeros, N, bias, res, act, y, bound) == ORC_OK);
    EXPECT(orc_w4_matmul_ep(x, M, K, Wq, scales, zeros, N, bias, NULL, 7, y, bound) == ORC_BAD_SHAPE);
    EXPECT(orc_gelu(0.0) == 0.0 && orc_silu(0.0) == 0.0);

    /* group-64 affine variant */
    float *Wg = xmalloc(sizeof(float) * KG * N);
    for (int i = 0; i < KG * N; ++i) Wg[i] = 0.02f * rnd();
    uint8_t *Wqg = xmalloc(KG * N / 2), *Pqg = xmalloc(KG * N / 2);
    float *sg = xmalloc(sizeof(float) * KG / 64 * N), *mg = xmalloc(sizeof(float) * KG / 64 * N);
    float *Psg = xmalloc(sizeof(float) * KG / 64 * N), *Pmg = xmalloc(sizeof(float) * KG / 64 * N);
    float *Whg = xmalloc(sizeof(float) * KG * N);
    EXPECT(orc_w4g_quantize_pack(Wg, KG, N, Wqg, sg, mg) == ORC_OK);
    EXPECT(orc_w4g_dequantize(Wqg, sg, mg, KG, N, Whg) == ORC_OK);
    EXPECT(orc_w4g_prepack_kmajor(Wqg, sg, mg, KG, N, Pqg, Psg, Pmg) == ORC_OK);
    EXPECT(orc_w4g_matmul(x, M, KG, Wqg, sg, mg, N, bias, y, bound) == ORC_OK);

    /* int8 head */
    const int ldq = V + 3;
    float *E = xmalloc(sizeof(float) * K * V), *Eh = xmalloc(sizeof(float) * K * V);
    for (int i = 0; i < K * V; ++i) E[i] = 0.02f * rnd();
    for (int k = 0; k < K; ++k) E[k * V + 4] = 0.0f;  /* a zero column */
    int8_t *Q = xmalloc((size_t)K * ldq);
    float *hs = xmalloc(sizeof(float) * V), *logits = xmalloc(sizeof(float) * V);
    double *lb = xmalloc(sizeof(double) * V);
    EXPECT(orc_i8_quantize_head(E, K, V, ldq, Q, hs) == ORC_OK);
    EXPECT(orc_i8_dequantize_head(Q, ldq, hs, K, V, Eh) == ORC_OK);
    EXPECT(orc_i8_head_logits(x, K, Q, ldq, hs, V, logits, lb) == ORC_OK);
    int64_t tokens[T] = {0, 3, V - 1, 7, 2};
    float *emb = xmalloc(sizeof(float) * T * K);
    EXPECT(orc_i8_embed(tokens, T, Q, ldq, hs, K, V, emb) == ORC_OK);
    tokens[3] = V;   /* out of range: a status, never an out-of-bounds read */
    EXPECT(orc_i8_embed(tokens, T, Q, ldq, hs, K, V, emb) == ORC_BAD_SHAPE);
    tokens[3] = -1;
    EXPECT(orc_i8_embed(tokens, T, Q, ldq, hs, K, V, emb) == ORC_BAD_SHAPE);

    orc_set_threads(2);
    EXPECT(orc_get_threads() >= 1);
    EXPECT(orc_w4_matmul(x, M, K, Wq, scales, zeros, N, bias, y, bound) == ORC_OK);

    free(W); free(x); free(bias); free(res); free(Wq); free(zeros); free(scales); free(What);
    free(q); free(z); free(Pq); free(Pz); free(Ps); free(y); free(bound); free(s16); free(s16f);
    free(Wg); free(Wqg); free(Pqg); free(sg); free(mg); free(Psg); free(Pmg); free(Whg);
    free(E); free(Eh); free(Q); free(hs); free(logits); free(lb); free(emb);
    if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
    return failures ? 1 : 0;
}
