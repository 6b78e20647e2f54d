// M > 1: the small-M path (prefill rows, batched decode).
#include "common.h"
#include "launch.h"

namespace w4 {

hipError_t launch_matmul_generic(const float *x, int64_t M, int64_t K, const uint8_t *Wq,
                                 const float *scales, const uint8_t *zeros, int64_t N,
                                 const float *bias, float *y, hipStream_t stream);

hipError_t launch_small_m(const SmallMPlan &p, const float *x, int64_t M, int64_t K,
                          const uint8_t *Wq, const float *scales, const uint8_t *zeros,
                          int64_t N, const float *bias, float *y, void *workspace,
                          hipStream_t stream) {
    (void)workspace;
    switch (p.kind) {
    case SmallMPlan::kEmpty:
        return hipSuccess;
    case SmallMPlan::kBiasOnly:
        return launch_bias_fill(bias, M, N, y, stream);
    default:
        return launch_matmul_generic(x, M, K, Wq, scales, zeros, N, bias, y, stream);
    }
}

}  // namespace w4
