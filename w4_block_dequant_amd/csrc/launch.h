// Kernel launchers (one per entry point).  Arguments are already validated;
// each launcher only enqueues work on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"
#include "splitk.h"

namespace w4 {

// scales are fp32, or binary16 bit patterns when f16 is set
hipError_t launch_quantize_pack(const float *W, int64_t K, int64_t N, uint8_t *Wq, void *scales,
                                bool f16, uint8_t *zeros, int *d_status, hipStream_t stream);
hipError_t launch_unpack(const uint8_t *Wq, const uint8_t *zeros, int64_t K, int64_t N,
                         uint8_t *q, uint8_t *z, hipStream_t stream);
hipError_t launch_dequantize(const uint8_t *Wq, const void *scales, bool f16,
                             const uint8_t *zeros, int64_t K, int64_t N, float *out,
                             hipStream_t stream);

hipError_t launch_gemv(const GemvPlan &plan, const float *x, int64_t K, const uint8_t *Wq,
                       const float *scales, const uint8_t *zeros, int64_t N, const float *bias,
                       float *y, void *workspace, hipStream_t stream);

hipError_t launch_small_m(const SmallMPlan &plan, const float *x, int64_t M, int64_t K,
                          const uint8_t *Wq, const float *scales, const uint8_t *zeros,
                          int64_t N, const float *bias, float *y, void *workspace,
                          hipStream_t stream);

hipError_t launch_prepack_kmajor(const uint8_t *Wq, const void *scales, bool f16,
                                 const uint8_t *zeros, int64_t K, int64_t N, uint8_t *Pq, void *Ps,
                                 uint8_t *Pz, hipStream_t stream);
hipError_t launch_gemv_kmajor(const KmajorPlan &plan, const float *x, int64_t M, int64_t K,
                              const uint8_t *Pq, const void *Ps, bool f16, const void *Pz,
                              int64_t N, const float *bias, const float *residual, int act,
                              float *y, hipStream_t stream, bool affine = false);
// Group-64 affine variant: quantize + pack, dequantize, K-major copy.
hipError_t launch_g64_quantize_pack(const float *W, int64_t K, int64_t N, uint8_t *Wq,
                                    float *scales, float *mins, int *d_status, hipStream_t stream);
hipError_t launch_g64_dequantize(const uint8_t *Wq, const float *scales, const float *mins,
                                 int64_t K, int64_t N, float *W_hat, hipStream_t stream);
hipError_t launch_prepack_g64(const uint8_t *Wq, const float *scales, const float *mins,
                              int64_t K, int64_t N, uint8_t *Pq, float *Ps, float *Pm,
                              hipStream_t stream);
// The fused epilogue alone (K = 0: the pre-activation values are the bias).
hipError_t launch_epilogue_only(const float *bias, int64_t M, int64_t N, const float *residual,
                                int act, float *y, hipStream_t stream);

hipError_t launch_bias_fill(const float *bias, int64_t M, int64_t N, float *y,
                            hipStream_t stream);

hipError_t launch_head_quantize(const float *E, int64_t K, int64_t N, int64_t ldq, int8_t *Q,
                                float *hs, int *d_status, hipStream_t stream);
hipError_t launch_head_logits(const HeadPlan &plan, const float *x, int64_t K, const int8_t *Q,
                              int64_t ldq, const float *hs, int64_t N, float *logits,
                              void *workspace, hipStream_t stream);
hipError_t launch_embed(const int64_t *tokens, int64_t T, const int8_t *Q, int64_t ldq,
                        const float *hs, int64_t K, int64_t N, float *out, int *d_status,
                        hipStream_t stream);
hipError_t launch_mm_x3(const X3Plan &p, const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                        const void *Ps, bool f16, const uint8_t *Pz, int64_t N, const float *bias,
                        const float *residual, int act, float *y, void *workspace,
                        hipStream_t stream);
hipError_t launch_head_prepack(const int8_t *Q, int64_t K, int64_t N, int64_t ldq, int8_t *Qt,
                               int64_t ldt, hipStream_t stream);
hipError_t launch_head_logits_kmajor(const float *x, int64_t K, const int8_t *Qt, int64_t ldt,
                                     const float *hs, int64_t N, float *logits,
                                     hipStream_t stream);
size_t head_rows_workspace(int64_t M, int64_t K);
hipError_t launch_head_rows_kmajor(const float *x, int64_t M, int64_t K, const int8_t *Qt,
                                  int64_t ldt, const float *hs, int64_t N, float *logits,
                                  void *workspace, hipStream_t stream);
hipError_t launch_embed_kmajor(const int64_t *tokens, int64_t T, const int8_t *Qt, int64_t ldt,
                               const float *hs, int64_t K, int64_t N, float *out, int *d_status,
                               hipStream_t stream);

// Streaming-read reference: `loads` 16-byte loads per lane, 256 lanes per
// workgroup, one XOR word per wave into out[read_bytes_words(...)].
int64_t read_bytes_groups(int64_t bytes, int loads);
int64_t read_bytes_words(int64_t bytes, int loads);
hipError_t launch_read_bytes(const void *src, int64_t bytes, int loads, uint32_t *out,
                             hipStream_t stream);

}  // namespace w4
