// Internal declarations shared by the HIP sources of libq2_0.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/q2_0.h"

namespace q2_0 {

constexpr int kBlockWeights = 64;
constexpr int kBlockBytes = 18;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// IEEE half bits -> f32 (v_cvt_f32_f16: exact for every half, subnormals included).
__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Scale and one 32-bit code word of block `blk` from a 2-byte aligned block base.
// Word w sits at byte 2 + 4w: 4-byte aligned only for odd blocks of an aligned row,
// so it is read as two half-words.
__device__ __forceinline__ uint32_t load_word_u16x2(const uint16_t *blk16, int w) {
    return (uint32_t)blk16[1 + 2 * w] | ((uint32_t)blk16[2 + 2 * w] << 16);
}

// Launchers (return the HIP error of the launch).
hipError_t launch_get_rows(const uint8_t *w, int64_t M, int nb, const int32_t *ids, int64_t n_ids,
                           float *out, int64_t ld_out, hipStream_t s);
hipError_t launch_mat_vec(const uint8_t *w, int64_t M, int nb, const float *x, int64_t ldx, int N,
                          float *y, int64_t ldy, hipStream_t s);
hipError_t launch_mat_vec_group(const q2_0_mat_vec_item *items, int64_t n_items, int nb,
                                const float *x, int64_t ldx, int N, hipStream_t s);
bool mat_vec_mfma_eligible(const uint8_t *w, int64_t M, int nb, const float *x, int64_t ldx);
hipError_t launch_mat_vec_mfma(const uint8_t *w, int64_t M, int nb, const float *x, int64_t ldx,
                               int N, float *y, int64_t ldy, hipStream_t s);
// fp16-MFMA GEMM over one or more matrices that share K and x.
struct GemmMat {
    const uint8_t *w;
    int64_t M;
    float *y;
    int64_t ldy;
};
constexpr int kGemmMaxGroup = 16;   // matrices per GEMM launch (kernel argument size)
struct GemmItem {
    const uint8_t *w;
    float *y;
    int64_t ldy;
    float *part;   // this matrix's split-K partials (splits x N x M floats)
    int M;
    int tm0;       // first row tile of this matrix, counted across the call
};
struct GemmGroup {
    GemmItem p[kGemmMaxGroup];
    int tm0[kGemmMaxGroup];   // p[i].tm0 contiguously; INT_MAX past n
    int n;
    int tm_base;              // first row tile of this launch
};
size_t gemm_f16_workspace_bytes(const int64_t *Ms, int64_t n_items, int64_t K, int64_t N);
hipError_t launch_gemm_f16_group(const GemmMat *mats, int64_t n_items, int nb, const float *x, int64_t ldx,
                                 int64_t N, void *workspace, hipStream_t s);
hipError_t launch_gemm_f32(const uint8_t *w, int64_t M, int nb, const float *x, int64_t ldx,
                           int64_t N, float *y, int64_t ldy, hipStream_t s);

}  // namespace q2_0
