// Measured ceilings of one MI355X (gfx950), for the roofline fractions of the Q2_0 kernels.
// This library (libq2_0_ceilings.so) is measurement code only: the product is libq2_0.so.
//
//   q2_0_ceil_read_stream  -- HBM read rate: every byte of a buffer read once with
//                             16-byte loads (grid-stride, U loads in flight per thread),
//                             nothing written but one word per workgroup.
//   q2_0_ceil_mfma_f16     -- dense fp16 matrix-core rate: v_mfma_f32_32x32x16_f16 on
//                             operands held in registers (no memory traffic in the loop),
//                             four independent accumulators per wave.
//   q2_0_ceil_empty        -- one workgroup that does nothing: the fixed cost of a launch.
//   q2_0_probe_mfma_f16    -- one v_mfma_f32_32x32x16_f16 on given operands: how the matrix
//                             cores round (the fp32-grade GEMM's error bound counts on it).
//
// All return the hipError_t of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

template <int U, bool NT>
__global__ __launch_bounds__(1024) void read_stream(const u32x4_t *__restrict__ p, int64_t n16,
                                                    uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4_t v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // the loads feed this value, so they cannot be dropped; one word per workgroup
    acc ^= __shfl_xor(acc, 1);
    if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void mfma_f16_loop(int iters, float *__restrict__ out, uint32_t seed) {
    // operands: pseudo-random fp16 values in [-1, 1) per lane (a fixed hash of lane and seed)
    half8_t a, b;
    uint32_t h = (threadIdx.x + 1u) * 2654435761u ^ seed;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h = h * 1664525u + 1013904223u;
        a[e] = (_Float16)((float)(h >> 8) * (1.0f / 8388608.0f) - 1.0f);
        h = h * 1664525u + 1013904223u;
        b[e] = (_Float16)((float)(h >> 8) * (1.0f / 8388608.0f) - 1.0f);
    }
    float16_t acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
    for (int it = 0; it < iters; ++it) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, acc1, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, acc2, 0, 0, 0);
        acc3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, b, acc3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc0[e] + acc1[e] + acc2[e] + acc3[e];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void empty_kernel() {}

// One wave: every row of A and every column of B carry the same 16 k-values a16[k] and
// b16[k] (lane l holds k = 8 (l / 32) .. + 7, the layout of both operands), every
// accumulator element starts at c; out receives the 16 results of every lane.
__global__ __launch_bounds__(64) void mfma_f16_probe(const _Float16 *a16, const _Float16 *b16, float c, float *out) {
    const int lane = threadIdx.x;
    half8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = a16[8 * (lane / 32) + e];
        b[e] = b16[8 * (lane / 32) + e];
    }
    float16_t acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = c;
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 16; ++v) out[lane * 16 + v] = acc[v];
}

}  // namespace

extern "C" {

// Reads bytes (a multiple of 16) at p once.  threads: workgroup size (64..1024, a multiple of
// 64); grid: workgroups; unroll: loads in flight per thread (1, 2, 4 or 8); nontemporal: 1 for
// streaming (non-temporal) loads.  sink: grid words of device memory.
int q2_0_ceil_read_stream(const void *p, int64_t bytes, void *sink, int threads, int grid, int unroll,
                          int nontemporal, void *stream) {
    if (!p || !sink || bytes <= 0 || bytes % 16 || threads < 64 || threads > 1024 || threads % 64 || grid < 1)
        return (int)hipErrorInvalidValue;
    const u32x4_t *q = static_cast<const u32x4_t *>(p);
    const int64_t n16 = bytes / 16;
    uint32_t *s = static_cast<uint32_t *>(sink);
    hipStream_t st = static_cast<hipStream_t>(stream);
#define Q2_0_CEIL_RS(U)                                                                             \
    do {                                                                                            \
        if (nontemporal)                                                                            \
            read_stream<U, true><<<grid, threads, 0, st>>>(q, n16, s);                              \
        else                                                                                        \
            read_stream<U, false><<<grid, threads, 0, st>>>(q, n16, s);                             \
    } while (0)
    switch (unroll) {
        case 1: Q2_0_CEIL_RS(1); break;
        case 2: Q2_0_CEIL_RS(2); break;
        case 4: Q2_0_CEIL_RS(4); break;
        case 8: Q2_0_CEIL_RS(8); break;
        default: return (int)hipErrorInvalidValue;
    }
#undef Q2_0_CEIL_RS
    return (int)hipGetLastError();
}

// grid workgroups of 256 threads, each wave running iters x 4 MFMAs of 32x32x16 (32768 flops
// each).  out: grid * 256 floats of device memory.
int q2_0_ceil_mfma_f16(int grid, int iters, void *out, void *stream) {
    if (!out || grid < 1 || iters < 1) return (int)hipErrorInvalidValue;
    mfma_f16_loop<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, static_cast<float *>(out), 12345u);
    return (int)hipGetLastError();
}

// a16, b16: 16 halves each; out: 1024 floats (device memory).  Synchronous.
int q2_0_probe_mfma_f16(const void *a16, const void *b16, float c, void *out) {
    if (!a16 || !b16 || !out) return (int)hipErrorInvalidValue;
    mfma_f16_probe<<<1, 64>>>(static_cast<const _Float16 *>(a16), static_cast<const _Float16 *>(b16), c,
                              static_cast<float *>(out));
    const hipError_t e = hipGetLastError();
    return (int)(e != hipSuccess ? e : hipDeviceSynchronize());
}

int q2_0_ceil_empty(void *stream) {
    empty_kernel<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>();
    return (int)hipGetLastError();
}

}  // extern "C"
