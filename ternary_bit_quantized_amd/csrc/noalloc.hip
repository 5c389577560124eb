// q2_0_mul_mat_noalloc: q2_0_mul_mat without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops).  The fp16
// GEMM's scratch (x as fp16, its column exponents, split-K partials) lives in one
// file-scope device array of Q2_0_NOALLOC_SCRATCH_BYTES, which every GPU the library runs
// on holds until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and only that address is ever handed to
// kernels.  All calls on one GPU share the array, so calls that overlap in time on one GPU
// race; nothing in it needs to start at zero (every kernel writes what it later reads).
#include <atomic>

#include "../../include/q2_0.h"
#include "q2_0_internal.h"

namespace {

__device__ __align__(256) uint8_t scratch[Q2_0_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];   // device address of `scratch` per device

// The current device's address of `scratch`, looked up on the first call on that device
// (threads racing here look up the same address).  nullptr and *err set on failure.
void *device_scratch(hipError_t *err) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" int q2_0_mul_mat_noalloc(const void *w, int64_t M, int64_t K, const float *x, int64_t ldx, int64_t N,
                                    float *y, int64_t ldy, int precision, void *stream) {
    bool noop;
    const int st = q2_0::check_mul_mat(w, M, K, x, Q2_0_ACT_F32, ldx, N, y, ldy, precision, &noop);
    if (st || noop) return st;
    const size_t need = q2_0_mul_mat_workspace_bytes(M, K, N, precision);
    if (need > Q2_0_NOALLOC_SCRATCH_BYTES) return Q2_0_ERR_TOO_LARGE;
    if (need == 0) return q2_0_mul_mat(w, M, K, x, ldx, N, y, ldy, precision, nullptr, 0, stream);
    hipError_t e;
    void *ws = device_scratch(&e);
    if (!ws) return q2_0::record_hip_error(e);
    return q2_0_mul_mat(w, M, K, x, ldx, N, y, ldy, precision, ws, Q2_0_NOALLOC_SCRATCH_BYTES, stream);
}
