// Deterministic split-K combination across workgroups.
//
// Each of the `splits` workgroups of a column tile stores its fp32 partial
// sums, then increments the tile's arrival counter.  The workgroup that
// arrives last reads every split's partials in split order (so the result
// does not depend on arrival order), writes the output and resets the
// counter to zero for the next launch.  No floating-point atomics.
#pragma once

#include "common.h"

namespace w4 {

// All threads of the workgroup call this after storing their partials.
// Returns true (in every thread) for the workgroup that must finish the tile.
__device__ __forceinline__ bool splitk_arrive(unsigned *counter, int64_t splits) {
    __shared__ int s_last;
    __threadfence();  // release: partials visible beyond this XCD's L2
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = atomicAdd(counter, 1u);
        s_last = (prev == (unsigned)(splits - 1));
    }
    __syncthreads();
    const bool last = s_last != 0;
    if (last) __threadfence();  // acquire: see every other split's partials
    return last;
}

__device__ __forceinline__ void splitk_reset(unsigned *counter) {
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace w4
