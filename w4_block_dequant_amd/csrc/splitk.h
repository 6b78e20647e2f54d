// Deterministic split-K combination across workgroups.
//
// Each of the `splits` workgroups of a column tile stores its fp32 partial
// sums, then increments the tile's arrival counter.  The workgroup that
// arrives last reads every split's partials in split order (so the result
// does not depend on arrival order), writes the output and resets the
// counter to zero for the next launch.  No floating-point atomics.
//
// Visibility across the XCDs (each has its own L2) is obtained without a
// device-scope fence, which on gfx950 writes back and invalidates the whole
// L2 of the calling XCD: the partials are written with device-scope stores
// (sc1, coherent at the device level) and read with device-scope loads, and
// every thread waits for its stores to complete (s_waitcnt) before the
// workgroup barrier that precedes the counter increment.  The last
// workgroup issues its loads only after its counter RMW has returned.
#pragma once

#include "common.h"

namespace w4 {

__device__ __forceinline__ void store_partial(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_partial(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// All threads of the workgroup call this after storing their partials with
// store_partial.  Returns true (in every thread) for the workgroup that must
// finish the tile.
__device__ __forceinline__ bool splitk_arrive(unsigned *counter, int64_t splits) {
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev =
            __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (unsigned)(splits - 1));
    }
    __syncthreads();
    return s_last != 0;
}

__device__ __forceinline__ void splitk_reset(unsigned *counter) {
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace w4
