// Fused epilogues of the K-major matmul (pages "rlx-web": a SwiGLU MLP;
// "zero-tvm": a fused gate + up + SiLU kernel and a fused residual add; the
// GELU is GPT-2's MLP activation in its tanh form).  Applied where each
// kernel stores its final value t = x . W_hat + bias:
//   W4_ACT_NONE    out[m, n] = t[m, n]
//   W4_ACT_GELU    out[m, n] = gelu(t[m, n])
//   W4_ACT_SWIGLU  out[m, i] = silu(t[m, 2 i]) * t[m, 2 i + 1]  (gate, up
//                  columns interleaved; the output has N / 2 columns)
// then + residual[m, n_out] when given.  fp32, with the device library's
// tanhf and expf.
#pragma once

#include "common.h"

namespace w4 {

__device__ __forceinline__ float ep_gelu(float v) {
    const float c = 0.7978845608028654f;  // sqrt(2 / pi)
    return 0.5f * v * (1.0f + tanhf(c * (v + 0.044715f * v * v * v)));
}

__device__ __forceinline__ float ep_silu(float v) { return v / (1.0f + expf(-v)); }

// Store of a non-SwiGLU output: activation, then the residual.
__device__ __forceinline__ void ep_store(float t, int act, const float *residual, float *y,
                                         size_t i) {
    float out = act == W4_ACT_GELU ? ep_gelu(t) : t;
    if (residual) out += residual[i];
    y[i] = out;
}

// Store of a SwiGLU output from its gate and up values.
__device__ __forceinline__ void ep_store_glu(float gate, float up, const float *residual,
                                             float *y, size_t i) {
    float out = ep_silu(gate) * up;
    if (residual) out += residual[i];
    y[i] = out;
}

}  // namespace w4
