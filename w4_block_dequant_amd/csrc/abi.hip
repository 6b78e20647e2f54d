// The C ABI (include/w4.h): host-side argument checks, device check, and
// dispatch to the kernel launchers.  Every check runs before any HIP call,
// so a rejected call enqueues nothing; the w4_check_* functions run the same
// checks with no HIP call at all.
#include <atomic>
#include <string.h>

#include "launch.h"
#include "w4.h"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;  // keeps every index in int64 range

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// A pointer is required unless the buffer it names is empty.
bool need(const void *p, int64_t count) { return count == 0 || p != nullptr; }

int check_w4_shape(int64_t K, int64_t N) {
    if (K < 0 || N < 0 || K % 32 != 0 || N % 2 != 0) return W4_ERR_BAD_SHAPE;
    if (K > kMaxElems / (N > 0 ? N : 1)) return W4_ERR_BAD_SHAPE;
    return W4_OK;
}

int check_packed(const uint8_t *Wq, const void *scales, const uint8_t *zeros, int64_t K,
                 int64_t N) {
    if (!need(Wq, K * N) || !need(scales, K * N) || !need(zeros, K * N)) return W4_ERR_NULL_PTR;
    if (!aligned(Wq, 16) || !aligned(scales, 16) || !aligned(zeros, 16)) return W4_ERR_MISALIGNED;
    return W4_OK;
}

size_t matmul_workspace(int64_t M, int64_t K, int64_t N) {
    if (M == 1) return w4::plan_gemv(K, N).workspace;
    return w4::plan_small_m(M, K, N).workspace;
}

// The current device must be a gfx950; the answer is cached per device.
int device_check() {
    static std::atomic<int> cache[64];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return W4_ERR_DEVICE;
    }
    if (dev >= 64) return W4_ERR_DEVICE;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return W4_ERR_DEVICE;
        }
        c = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        cache[dev].store(c, std::memory_order_relaxed);
    }
    return c == 1 ? W4_OK : W4_ERR_DEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? W4_OK : W4_ERR_LAUNCH; }

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int w4_abi_version(void) { return W4_ABI_VERSION; }

const char *w4_strerror(int status) {
    switch (status) {
    case W4_OK: return "ok";
    case W4_ERR_NULL_PTR: return "a required pointer is NULL";
    case W4_ERR_BAD_SHAPE: return "bad shape (negative size, K % 32 != 0, N odd, ldq < N, or token id out of range)";
    case W4_ERR_MISALIGNED: return "misaligned pointer";
    case W4_ERR_WORKSPACE: return "workspace missing or too small";
    case W4_ERR_DEVICE: return "no current HIP device, or the device is not gfx950";
    case W4_ERR_LAUNCH: return "kernel launch failed";
    case W4_ERR_NONFINITE: return "non-finite input value";
    default: return "unknown status";
    }
}

static int quantize_pack_impl(const float *W, int64_t K, int64_t N, uint8_t *Wq, void *scales, bool f16,
                       uint8_t *zeros, int *d_status, void *stream) {
    int st = check_w4_shape(K, N);
    if (st) return st;
    if (!need(W, K * N)) return W4_ERR_NULL_PTR;
    if ((st = check_packed(Wq, scales, zeros, K, N))) return st;
    if (!aligned(W, 16) || !aligned(d_status, 4)) return W4_ERR_MISALIGNED;
    if ((st = device_check())) return st;
    return launched(
        w4::launch_quantize_pack(W, K, N, Wq, scales, f16, zeros, d_status, as_stream(stream)));
}

int w4_quantize_pack(const float *W, int64_t K, int64_t N, uint8_t *Wq, float *scales,
                     uint8_t *zeros, int *d_status, void *stream) {
    return quantize_pack_impl(W, K, N, Wq, scales, false, zeros, d_status, stream);
}

int w4h_quantize_pack(const float *W, int64_t K, int64_t N, uint8_t *Wq, uint16_t *scales,
                      uint8_t *zeros, int *d_status, void *stream) {
    return quantize_pack_impl(W, K, N, Wq, scales, true, zeros, d_status, stream);
}

int w4_unpack(const uint8_t *Wq, const uint8_t *zeros, int64_t K, int64_t N, uint8_t *q,
              uint8_t *z, void *stream) {
    int st = check_w4_shape(K, N);
    if (st) return st;
    if (!need(Wq, K * N) || !need(zeros, K * N) || !need(q, K * N) || !need(z, K * N))
        return W4_ERR_NULL_PTR;
    if (!aligned(Wq, 16) || !aligned(zeros, 16) || !aligned(q, 2) || !aligned(z, 2))
        return W4_ERR_MISALIGNED;
    if ((st = device_check())) return st;
    return launched(w4::launch_unpack(Wq, zeros, K, N, q, z, as_stream(stream)));
}

static int dequantize_impl(const uint8_t *Wq, const void *scales, bool f16, const uint8_t *zeros,
                    int64_t K, int64_t N, float *W_hat, void *stream) {
    int st = check_w4_shape(K, N);
    if (st) return st;
    if ((st = check_packed(Wq, scales, zeros, K, N))) return st;
    if (!need(W_hat, K * N)) return W4_ERR_NULL_PTR;
    if (!aligned(W_hat, 8)) return W4_ERR_MISALIGNED;
    if ((st = device_check())) return st;
    return launched(
        w4::launch_dequantize(Wq, scales, f16, zeros, K, N, W_hat, as_stream(stream)));
}

int w4_dequantize(const uint8_t *Wq, const float *scales, const uint8_t *zeros, int64_t K,
                  int64_t N, float *W_hat, void *stream) {
    return dequantize_impl(Wq, scales, false, zeros, K, N, W_hat, stream);
}

int w4h_dequantize(const uint8_t *Wq, const uint16_t *scales, const uint8_t *zeros, int64_t K,
                   int64_t N, float *W_hat, void *stream) {
    return dequantize_impl(Wq, scales, true, zeros, K, N, W_hat, stream);
}

size_t w4_matmul_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M < 0 || check_w4_shape(K, N) != W4_OK) return 0;
    return matmul_workspace(M, K, N);
}

int w4_check_matmul_args(const float *x, int64_t M, int64_t K, const uint8_t *Wq,
                         const float *scales, const uint8_t *zeros, int64_t N, const float *bias,
                         const float *y, const void *workspace, size_t workspace_bytes) {
    if (M < 0) return W4_ERR_BAD_SHAPE;
    int st = check_w4_shape(K, N);
    if (st) return st;
    if (M > kMaxElems / (K > 0 ? K : 1) || M > kMaxElems / (N > 0 ? N : 1)) return W4_ERR_BAD_SHAPE;
    if (M == 0 || N == 0) return W4_OK;
    if (!need(x, M * K) || !y) return W4_ERR_NULL_PTR;
    if ((st = check_packed(Wq, scales, zeros, K, N))) return st;
    if (!aligned(x, 16) || !aligned(y, 4) || !aligned(bias, 4)) return W4_ERR_MISALIGNED;
    const size_t need_ws = matmul_workspace(M, K, N);
    if (need_ws > 0 && (workspace == nullptr || workspace_bytes < need_ws)) return W4_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return W4_ERR_MISALIGNED;
    return W4_OK;
}

int w4_matmul(const float *x, int64_t M, int64_t K, const uint8_t *Wq, const float *scales,
              const uint8_t *zeros, int64_t N, const float *bias, float *y, void *workspace,
              size_t workspace_bytes, void *stream) {
    int st = w4_check_matmul_args(x, M, K, Wq, scales, zeros, N, bias, y, workspace,
                                  workspace_bytes);
    if (st) return st;
    if (M == 0 || N == 0) return W4_OK;
    if ((st = device_check())) return st;
    if (M == 1)
        return launched(w4::launch_gemv(w4::plan_gemv(K, N), x, K, Wq, scales, zeros, N, bias, y,
                                        workspace, as_stream(stream)));
    return launched(w4::launch_small_m(w4::plan_small_m(M, K, N), x, M, K, Wq, scales, zeros, N,
                                       bias, y, workspace, as_stream(stream)));
}

static int prepack_kmajor_impl(const uint8_t *Wq, const void *scales, bool f16, const uint8_t *zeros,
                        int64_t K, int64_t N, uint8_t *Pq, void *Ps, uint8_t *Pz, void *stream) {
    int st = check_w4_shape(K, N);
    if (st) return st;
    if (K % 64 != 0) return W4_ERR_BAD_SHAPE;
    if ((st = check_packed(Wq, scales, zeros, K, N))) return st;
    if ((st = check_packed(Pq, Ps, Pz, K, N))) return st;
    if (K * N == 0) return W4_OK;
    if ((st = device_check())) return st;
    return launched(w4::launch_prepack_kmajor(Wq, scales, f16, zeros, K, N, Pq, Ps, Pz,
                                              as_stream(stream)));
}

int w4_prepack_kmajor(const uint8_t *Wq, const float *scales, const uint8_t *zeros, int64_t K,
                      int64_t N, uint8_t *Pq, float *Ps, uint8_t *Pz, void *stream) {
    return prepack_kmajor_impl(Wq, scales, false, zeros, K, N, Pq, Ps, Pz, stream);
}

int w4h_prepack_kmajor(const uint8_t *Wq, const uint16_t *scales, const uint8_t *zeros, int64_t K,
                       int64_t N, uint8_t *Pq, uint16_t *Ps, uint8_t *Pz, void *stream) {
    return prepack_kmajor_impl(Wq, scales, true, zeros, K, N, Pq, Ps, Pz, stream);
}

size_t w4_matmul_kmajor_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M < 0 || K < 0 || N < 0) return 0;
    return w4::plan_x3(M, K, N).workspace;
}

static int check_matmul_kmajor_impl(const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                                    const void *Ps, const uint8_t *Pz, int64_t N,
                                    const float *bias, const float *y, const void *workspace,
                                    size_t workspace_bytes, const float *residual = nullptr,
                                    int act = W4_ACT_NONE) {
    if (M < 0) return W4_ERR_BAD_SHAPE;
    if (act != W4_ACT_NONE && act != W4_ACT_GELU && act != W4_ACT_SWIGLU) return W4_ERR_BAD_SHAPE;
    int st = check_w4_shape(K, N);
    if (st) return st;
    if (K % 64 != 0) return W4_ERR_BAD_SHAPE;
    if (M > kMaxElems / (K > 0 ? K : 1) || M > kMaxElems / (N > 0 ? N : 1)) return W4_ERR_BAD_SHAPE;
    if (M == 0 || N == 0) return W4_OK;
    // the K-major kernels index with 32-bit offsets
    if (K * N >= ((int64_t)1 << 31) || M * K >= ((int64_t)1 << 31) || M * N >= ((int64_t)1 << 31))
        return W4_ERR_BAD_SHAPE;
    if (!need(x, M * K) || !y) return W4_ERR_NULL_PTR;
    if ((st = check_packed(Pq, Ps, Pz, K, N))) return st;
    if (!aligned(x, 16) || !aligned(y, 4) || !aligned(bias, 4) || !aligned(residual, 4))
        return W4_ERR_MISALIGNED;
    // off the matrix cores the GEMV takes rows in groups of 4 on the grid's y axis
    if (w4::plan_x3(M, K, N).kind == w4::X3Plan::kNone && (M + 3) / 4 > 65535)
        return W4_ERR_BAD_SHAPE;
    const size_t need_ws = w4::plan_x3(M, K, N).workspace;
    if (need_ws > 0 && (workspace == nullptr || workspace_bytes < need_ws)) return W4_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return W4_ERR_MISALIGNED;
    return W4_OK;
}

static int matmul_kmajor_impl(const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                              const void *Ps, bool f16, const uint8_t *Pz, int64_t N,
                              const float *bias, float *y, void *workspace,
                              size_t workspace_bytes, void *stream,
                              const float *residual = nullptr, int act = W4_ACT_NONE) {
    int st = check_matmul_kmajor_impl(x, M, K, Pq, Ps, Pz, N, bias, y, workspace,
                                      workspace_bytes, residual, act);
    if (st) return st;
    if (M == 0 || N == 0) return W4_OK;
    if ((st = device_check())) return st;
    const w4::X3Plan px = w4::plan_x3(M, K, N);
    if (K > 0 && px.kind != w4::X3Plan::kNone)
        return launched(w4::launch_mm_x3(px, x, M, K, Pq, Ps, f16, Pz, N, bias, residual, act, y,
                                         workspace, as_stream(stream)));
    return launched(w4::launch_gemv_kmajor(w4::plan_kmajor(M, K, N, act == W4_ACT_SWIGLU), x, M,
                                           K, Pq, Ps, f16, Pz, N, bias, residual, act, y,
                                           as_stream(stream)));
}

int w4_check_matmul_kmajor_args(const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                                const float *Ps, const uint8_t *Pz, int64_t N, const float *bias,
                                const float *y, const void *workspace, size_t workspace_bytes) {
    return check_matmul_kmajor_impl(x, M, K, Pq, Ps, Pz, N, bias, y, workspace, workspace_bytes);
}

int w4h_check_matmul_kmajor_args(const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                                 const uint16_t *Ps, const uint8_t *Pz, int64_t N,
                                 const float *bias, const float *y, const void *workspace,
                                 size_t workspace_bytes) {
    return check_matmul_kmajor_impl(x, M, K, Pq, Ps, Pz, N, bias, y, workspace, workspace_bytes);
}

int w4_matmul_kmajor(const float *x, int64_t M, int64_t K, const uint8_t *Pq, const float *Ps,
                     const uint8_t *Pz, int64_t N, const float *bias, float *y, void *workspace,
                     size_t workspace_bytes, void *stream) {
    return matmul_kmajor_impl(x, M, K, Pq, Ps, false, Pz, N, bias, y, workspace, workspace_bytes,
                              stream);
}

int w4h_matmul_kmajor(const float *x, int64_t M, int64_t K, const uint8_t *Pq, const uint16_t *Ps,
                      const uint8_t *Pz, int64_t N, const float *bias, float *y, void *workspace,
                      size_t workspace_bytes, void *stream) {
    return matmul_kmajor_impl(x, M, K, Pq, Ps, true, Pz, N, bias, y, workspace, workspace_bytes,
                              stream);
}

int w4_check_matmul_kmajor_ep_args(const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                                   const float *Ps, const uint8_t *Pz, int64_t N,
                                   const float *bias, const float *residual, int act,
                                   const float *y, const void *workspace,
                                   size_t workspace_bytes) {
    return check_matmul_kmajor_impl(x, M, K, Pq, Ps, Pz, N, bias, y, workspace, workspace_bytes,
                                    residual, act);
}

int w4_matmul_kmajor_ep(const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                        const float *Ps, const uint8_t *Pz, int64_t N, const float *bias,
                        const float *residual, int act, float *y, void *workspace,
                        size_t workspace_bytes, void *stream) {
    return matmul_kmajor_impl(x, M, K, Pq, Ps, false, Pz, N, bias, y, workspace, workspace_bytes,
                              stream, residual, act);
}

// ---- group-64 affine variant ------------------------------------------------
static int check_g64_shape(int64_t K, int64_t N) {
    if (K < 0 || N < 0 || K % 64 != 0 || N % 2 != 0) return W4_ERR_BAD_SHAPE;
    if (K > kMaxElems / (N > 0 ? N : 1)) return W4_ERR_BAD_SHAPE;
    return W4_OK;
}

static int check_g64_packed(const uint8_t *Wq, const float *scales, const float *mins, int64_t K,
                            int64_t N) {
    if (!need(Wq, K * N) || !need(scales, K * N) || !need(mins, K * N)) return W4_ERR_NULL_PTR;
    if (!aligned(Wq, 16) || !aligned(scales, 16) || !aligned(mins, 16)) return W4_ERR_MISALIGNED;
    return W4_OK;
}

int w4g_quantize_pack(const float *W, int64_t K, int64_t N, uint8_t *Wq, float *scales,
                      float *mins, int *d_status, void *stream) {
    int st = check_g64_shape(K, N);
    if (st) return st;
    if (!need(W, K * N)) return W4_ERR_NULL_PTR;
    if ((st = check_g64_packed(Wq, scales, mins, K, N))) return st;
    if (!aligned(W, 16) || !aligned(d_status, 4)) return W4_ERR_MISALIGNED;
    if ((st = device_check())) return st;
    return launched(
        w4::launch_g64_quantize_pack(W, K, N, Wq, scales, mins, d_status, as_stream(stream)));
}

int w4g_dequantize(const uint8_t *Wq, const float *scales, const float *mins, int64_t K,
                   int64_t N, float *W_hat, void *stream) {
    int st = check_g64_shape(K, N);
    if (st) return st;
    if ((st = check_g64_packed(Wq, scales, mins, K, N))) return st;
    if (!need(W_hat, K * N)) return W4_ERR_NULL_PTR;
    if (!aligned(W_hat, 8)) return W4_ERR_MISALIGNED;
    if ((st = device_check())) return st;
    return launched(w4::launch_g64_dequantize(Wq, scales, mins, K, N, W_hat, as_stream(stream)));
}

int w4g_prepack_kmajor(const uint8_t *Wq, const float *scales, const float *mins, int64_t K,
                       int64_t N, uint8_t *Pq, float *Ps, float *Pm, void *stream) {
    int st = check_g64_shape(K, N);
    if (st) return st;
    if ((st = check_g64_packed(Wq, scales, mins, K, N))) return st;
    if ((st = check_g64_packed(Pq, Ps, Pm, K, N))) return st;
    if ((st = device_check())) return st;
    return launched(
        w4::launch_prepack_g64(Wq, scales, mins, K, N, Pq, Ps, Pm, as_stream(stream)));
}

int w4g_check_matmul_kmajor_args(const float *x, int64_t M, int64_t K, const uint8_t *Pq,
                                 const float *Ps, const float *Pm, int64_t N, const float *bias,
                                 const float *y) {
    if (M < 0) return W4_ERR_BAD_SHAPE;
    int st = check_g64_shape(K, N);
    if (st) return st;
    if (M > kMaxElems / (K > 0 ? K : 1) || M > kMaxElems / (N > 0 ? N : 1)) return W4_ERR_BAD_SHAPE;
    if (M == 0 || N == 0) return W4_OK;
    if (K * N >= ((int64_t)1 << 31) || M * K >= ((int64_t)1 << 31) || M * N >= ((int64_t)1 << 31))
        return W4_ERR_BAD_SHAPE;
    if ((M + 3) / 4 > 65535) return W4_ERR_BAD_SHAPE;
    if (!need(x, M * K) || !y) return W4_ERR_NULL_PTR;
    if ((st = check_g64_packed(Pq, Ps, Pm, K, N))) return st;
    if (!aligned(x, 16) || !aligned(y, 4) || !aligned(bias, 4)) return W4_ERR_MISALIGNED;
    return W4_OK;
}

int w4g_matmul_kmajor(const float *x, int64_t M, int64_t K, const uint8_t *Pq, const float *Ps,
                      const float *Pm, int64_t N, const float *bias, float *y, void *stream) {
    int st = w4g_check_matmul_kmajor_args(x, M, K, Pq, Ps, Pm, N, bias, y);
    if (st) return st;
    if (M == 0 || N == 0) return W4_OK;
    if ((st = device_check())) return st;
    return launched(w4::launch_gemv_kmajor(w4::plan_kmajor(M, K, N), x, M, K, Pq, Ps, false, Pm,
                                           N, bias, nullptr, W4_ACT_NONE, y, as_stream(stream),
                                           true));
}

int i8_quantize_head(const float *E, int64_t K, int64_t N, int64_t ldq, int8_t *Q, float *hs,
                     int *d_status, void *stream) {
    if (K < 0 || N < 0 || ldq < N) return W4_ERR_BAD_SHAPE;
    if (K > kMaxElems / (ldq > 0 ? ldq : 1)) return W4_ERR_BAD_SHAPE;
    if (!need(E, K * N) || !need(Q, K * ldq) || !need(hs, N)) return W4_ERR_NULL_PTR;
    if (!aligned(E, 4) || !aligned(Q, 16) || !aligned(hs, 4) || !aligned(d_status, 4))
        return W4_ERR_MISALIGNED;
    if (K * ldq == 0 && N == 0) return W4_OK;
    int st = device_check();
    if (st) return st;
    return launched(w4::launch_head_quantize(E, K, N, ldq, Q, hs, d_status, as_stream(stream)));
}

size_t i8_head_workspace_bytes(int64_t K, int64_t N) {
    if (K < 0 || N < 0) return 0;
    return w4::plan_head(K, N).workspace;
}

int i8_head_logits(const float *x_last, int64_t K, const int8_t *Q, int64_t ldq, const float *hs,
                   int64_t N, float *logits, void *workspace, size_t workspace_bytes,
                   void *stream) {
    if (K < 0 || N < 0 || ldq < N) return W4_ERR_BAD_SHAPE;
    if (K > kMaxElems / (ldq > 0 ? ldq : 1)) return W4_ERR_BAD_SHAPE;
    if (N == 0) return W4_OK;
    if (!need(x_last, K) || !need(Q, K * ldq) || !hs || !logits) return W4_ERR_NULL_PTR;
    if (!aligned(x_last, 4) || !aligned(Q, 16) || !aligned(hs, 4) || !aligned(logits, 4))
        return W4_ERR_MISALIGNED;
    const w4::HeadPlan plan = w4::plan_head(K, N);
    if (plan.workspace > 0 && (workspace == nullptr || workspace_bytes < plan.workspace))
        return W4_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return W4_ERR_MISALIGNED;
    int st = device_check();
    if (st) return st;
    return launched(w4::launch_head_logits(plan, x_last, K, Q, ldq, hs, N, logits, workspace,
                                           as_stream(stream)));
}

int i8_embed(const int64_t *tokens, int64_t T, const int8_t *Q, int64_t ldq, const float *hs,
             int64_t K, int64_t N, float *out, int *d_status, void *stream) {
    if (T < 0 || K < 0 || N < 0 || ldq < N) return W4_ERR_BAD_SHAPE;
    if (K > kMaxElems / (ldq > 0 ? ldq : 1) || T > kMaxElems / (K > 0 ? K : 1))
        return W4_ERR_BAD_SHAPE;
    if (T * K == 0) return W4_OK;
    if (!tokens || !Q || !hs || !out) return W4_ERR_NULL_PTR;
    if (!aligned(tokens, 8) || !aligned(Q, 16) || !aligned(hs, 4) || !aligned(out, 4) ||
        !aligned(d_status, 4))
        return W4_ERR_MISALIGNED;
    int st = device_check();
    if (st) return st;
    return launched(w4::launch_embed(tokens, T, Q, ldq, hs, K, N, out, d_status, as_stream(stream)));
}

int i8_prepack_head(const int8_t *Q, int64_t K, int64_t N, int64_t ldq, int8_t *Qt,
                    int64_t ldt, void *stream) {
    if (K < 0 || N < 0 || ldq < N || ldt < K || ldt % 16 != 0) return W4_ERR_BAD_SHAPE;
    if (K > kMaxElems / (ldq > 0 ? ldq : 1) || N > kMaxElems / (ldt > 0 ? ldt : 1) ||
        (ldt + 63) / 64 > 65535)
        return W4_ERR_BAD_SHAPE;
    if (N == 0 || ldt == 0) return W4_OK;
    if (!need(Q, K * ldq) || !Qt) return W4_ERR_NULL_PTR;
    if (!aligned(Q, 16) || !aligned(Qt, 16)) return W4_ERR_MISALIGNED;
    int st = device_check();
    if (st) return st;
    return launched(w4::launch_head_prepack(Q, K, N, ldq, Qt, ldt, as_stream(stream)));
}

int i8_check_head_logits_kmajor_args(const float *x_last, int64_t K, const int8_t *Qt,
                                     int64_t ldt, const float *hs, int64_t N,
                                     const float *logits) {
    if (K < 16 || K % 16 != 0 || K > 8192 || N < 0 || ldt < K || ldt % 16 != 0)
        return W4_ERR_BAD_SHAPE;
    if (N > 0 && N > ((int64_t)1 << 31) / ldt - 1) return W4_ERR_BAD_SHAPE;
    if (N == 0) return W4_OK;
    if (!x_last || !Qt || !hs || !logits) return W4_ERR_NULL_PTR;
    if (!aligned(x_last, 16) || !aligned(Qt, 16) || !aligned(hs, 4) || !aligned(logits, 4))
        return W4_ERR_MISALIGNED;
    return W4_OK;
}

int i8_head_logits_kmajor(const float *x_last, int64_t K, const int8_t *Qt, int64_t ldt,
                          const float *hs, int64_t N, float *logits, void *stream) {
    int st = i8_check_head_logits_kmajor_args(x_last, K, Qt, ldt, hs, N, logits);
    if (st) return st;
    if (N == 0) return W4_OK;
    if ((st = device_check())) return st;
    return launched(
        w4::launch_head_logits_kmajor(x_last, K, Qt, ldt, hs, N, logits, as_stream(stream)));
}

size_t i8_head_rows_workspace_bytes(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0) return 0;
    return w4::head_rows_workspace(M, K);
}

int i8_check_head_logits_rows_args(const float *x, int64_t M, int64_t K, const int8_t *Qt,
                                   int64_t ldt, const float *hs, int64_t N, const float *logits,
                                   const void *workspace, size_t workspace_bytes) {
    (void)workspace;
    (void)workspace_bytes;
    if (M < 0 || K < 16 || K % 16 != 0 || K > 8192 || N < 0 || ldt < K || ldt % 16 != 0)
        return W4_ERR_BAD_SHAPE;
    if (N > 0 && N > ((int64_t)1 << 31) / ldt - 1) return W4_ERR_BAD_SHAPE;
    if (M > 0 && (M > kMaxElems / K || M > kMaxElems / (N > 0 ? N : 1))) return W4_ERR_BAD_SHAPE;
    if (M == 0 || N == 0) return W4_OK;
    if (!x || !Qt || !hs || !logits) return W4_ERR_NULL_PTR;
    if (!aligned(x, 16) || !aligned(Qt, 16) || !aligned(hs, 4) || !aligned(logits, 4))
        return W4_ERR_MISALIGNED;
    return W4_OK;
}

int i8_head_logits_rows(const float *x, int64_t M, int64_t K, const int8_t *Qt, int64_t ldt,
                        const float *hs, int64_t N, float *logits, void *workspace,
                        size_t workspace_bytes, void *stream) {
    int st = i8_check_head_logits_rows_args(x, M, K, Qt, ldt, hs, N, logits, workspace,
                                            workspace_bytes);
    if (st) return st;
    if (M == 0 || N == 0) return W4_OK;
    if ((st = device_check())) return st;
    return launched(w4::launch_head_rows_kmajor(x, M, K, Qt, ldt, hs, N, logits, workspace,
                                                as_stream(stream)));
}

int i8_embed_kmajor(const int64_t *tokens, int64_t T, const int8_t *Qt, int64_t ldt,
                    const float *hs, int64_t K, int64_t N, float *out, int *d_status,
                    void *stream) {
    if (T < 0 || K < 0 || N < 0 || ldt < K || ldt % 16 != 0) return W4_ERR_BAD_SHAPE;
    if (N > kMaxElems / (ldt > 0 ? ldt : 1) || T > kMaxElems / (K > 0 ? K : 1))
        return W4_ERR_BAD_SHAPE;
    if (T * K == 0) return W4_OK;
    if (!tokens || !Qt || !hs || !out) return W4_ERR_NULL_PTR;
    if (!aligned(tokens, 8) || !aligned(Qt, 16) || !aligned(hs, 4) || !aligned(out, 4) ||
        !aligned(d_status, 4))
        return W4_ERR_MISALIGNED;
    int st = device_check();
    if (st) return st;
    return launched(
        w4::launch_embed_kmajor(tokens, T, Qt, ldt, hs, K, N, out, d_status, as_stream(stream)));
}

size_t w4_read_bytes_words(int64_t bytes, int loads_per_lane) {
    if (bytes <= 0 || bytes % 16 != 0) return 0;
    if (loads_per_lane != 4 && loads_per_lane != 6 && loads_per_lane != 8 &&
        loads_per_lane != 12 && loads_per_lane != 16)
        return 0;
    return (size_t)w4::read_bytes_words(bytes, loads_per_lane);
}

int w4_read_bytes(const void *src, int64_t bytes, int loads_per_lane, uint32_t *out,
                  void *stream) {
    if (bytes < 0 || bytes % 16 != 0) return W4_ERR_BAD_SHAPE;
    if (bytes == 0) return W4_OK;
    if (w4_read_bytes_words(bytes, loads_per_lane) == 0) return W4_ERR_BAD_SHAPE;
    if ((uint64_t)w4_read_bytes_words(bytes, loads_per_lane) > 0x7FFFFFFFu) return W4_ERR_BAD_SHAPE;
    if (!src || !out) return W4_ERR_NULL_PTR;
    if (!aligned(src, 16) || !aligned(out, 4)) return W4_ERR_MISALIGNED;
    int st = device_check();
    if (st) return st;
    return launched(w4::launch_read_bytes(src, bytes, loads_per_lane, out, as_stream(stream)));
}

}  // extern "C"
