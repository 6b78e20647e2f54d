// w4_matmul without any allocation (include/w4.h, w4_matmul_noalloc): the
// same kernels as w4_matmul, with the split-K partial sums in a fixed
// device array of this library instead of a caller workspace.
//
// `scratch` lives in device memory for the life of the process, one copy per
// GPU.  Host code never passes the array's name to a kernel or a copy: the
// name is a host-side stand-in.  The device address of each GPU's copy is
// looked up once per device (hipGetSymbolAddress with that device current)
// and cached; every later call on that device passes the cached address.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "w4.h"

namespace {

constexpr size_t kScratchBytes = (size_t)W4_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void *> g_addr[kMaxDevices];
std::mutex g_init;

// Device address of the current device's `scratch`, or nullptr on failure.
void *scratch_address(int dev) {
    void *p = g_addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_init);
    p = g_addr[dev].load(std::memory_order_relaxed);
    if (p) return p;
    void *q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) {
        (void)hipGetLastError();
        return nullptr;
    }
    g_addr[dev].store(q, std::memory_order_release);
    return q;
}

}  // namespace

extern "C" int w4_matmul_noalloc(const float *x, int64_t M, int64_t K, const uint8_t *Wq,
                                 const float *scales, const uint8_t *zeros, int64_t N,
                                 const float *bias, float *y, void *stream) {
    // host checks first, with a stand-in for the scratch (never dereferenced)
    int st = w4_check_matmul_args(x, M, K, Wq, scales, zeros, N, bias, y,
                                  reinterpret_cast<const void *>(kScratchBytes), kScratchBytes);
    if (st) return st;
    if (w4_matmul_workspace_bytes(M, K, N) > kScratchBytes) return W4_ERR_WORKSPACE;
    if (M == 0 || N == 0) return W4_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return W4_ERR_DEVICE;
    }
    void *ws = scratch_address(dev);
    if (!ws) return W4_ERR_DEVICE;
    return w4_matmul(x, M, K, Wq, scales, zeros, N, bias, y, ws, kScratchBytes, stream);
}
