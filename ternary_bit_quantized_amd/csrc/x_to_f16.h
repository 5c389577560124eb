// x -> fp16 for the GEMMs: one column per 256 threads, k permuted inside each 16-group.
// Shared by the GEMM's own conversion kernel (gemm_f16.hip) and the expert product's
// routing launch (mul_mat_id.hip), which converts the tokens' rows beside the routing.
#pragma once

#include "q2_0_internal.h"
#include "mat_vec_common.h"

namespace q2_0 {

// x (N columns of K floats) -> fp16, k permuted inside each 16-group, 256 threads per
// column.  The column is scaled by 2^e (e = xe[n]) so that its max |x| lands in
// [2^14, 2^15): fp16 then neither overflows (|x| > 65504) nor falls into its
// subnormal range, where the relative error would exceed 2^-11.  The GEMM multiplies
// the column's results by 2^-e.  Up to kPreGroups 16-value groups per thread are held
// in registers between the max and the conversion (x is read once); longer columns
// are read twice.
constexpr int kPreGroups = 4;

template <typename XT>
__device__ __forceinline__ void load16(const XT *src, bool vec, float v[16]) {
    if (vec) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4_t t = load_act4(src + 4 * q);
            v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = act_to_f32(src[q]);
    }
}

// HL: also the low halves lo = fp16(v - hi) at dst16 + lo_off (v - hi is exact in f32:
// hi is v rounded to 11 significant bits).
template <bool HL>
__device__ __forceinline__ void store16_perm(const float v[16], int e, _Float16 *dst16, int64_t lo_off) {
    uint32_t o[8], l[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const float a = __builtin_amdgcn_ldexpf(v[s], e), b = __builtin_amdgcn_ldexpf(v[s + 8], e);
        const _Float16 ha = (_Float16)a, hb = (_Float16)b;
        o[s] = __builtin_bit_cast(uint32_t, half2_t{ha, hb});
        if (HL) l[s] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)(a - (float)ha), (_Float16)(b - (float)hb)});
    }
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(dst16);
    dst[0] = u32x4_t{o[0], o[1], o[2], o[3]};
    dst[1] = u32x4_t{o[4], o[5], o[6], o[7]};
    if (HL) {
        u32x4_t *dl = reinterpret_cast<u32x4_t *>(dst16 + lo_off);
        dl[0] = u32x4_t{l[0], l[1], l[2], l[3]};
        dl[1] = u32x4_t{l[4], l[5], l[6], l[7]};
    }
}

// gather (expert routing): output column n converts x column of pair perm[n] (pair
// p = t * n_used + u reads column t when x_slots == 1, else column p).
struct XGather {
    const int *perm;   // nullptr: column n is x column n
    int n_used;
    int x_slots;
};

// Column n of x16 (HL: and its low halves lo_off halves further) and xe[n], by the 256
// threads tid = 0..255 of a workgroup part; red: 4 floats of LDS private to the part.
// The workgroup barrier inside is reached by every thread of the workgroup whether its
// part is active or not, so parts with and without a column may share a workgroup.
template <bool kVec, typename XT, bool HL>
__device__ __forceinline__ void convert_column(bool active, const XT *__restrict__ x, int64_t ldx, int K,
                                               _Float16 *__restrict__ x16, int *__restrict__ xe,
                                               const XGather &gather, int64_t lo_off, int64_t n, int tid,
                                               float *red) {
    int64_t src_col = n;
    if (active && gather.perm) {
        const int p = gather.perm[n];
        src_col = gather.x_slots == 1 ? p / gather.n_used : p;
    }
    const XT *col = x + src_col * ldx;
    const int groups = active ? K / 16 : 0;
    const bool resident = groups <= kPreGroups * 256;
    float v[kPreGroups][16];
    float m = 0.f;
    if (resident) {
#pragma unroll
        for (int u = 0; u < kPreGroups; ++u) {
            const int gi = tid + 256 * u;
            if (gi < groups) {
                load16(col + 16 * gi, kVec, v[u]);
#pragma unroll
                for (int q = 0; q < 16; ++q) m = fmaxf(m, fabsf(v[u][q]));
            }
        }
    } else {
        for (int gi = tid; gi < groups; gi += 256) {
            float t[16];
            load16(col + 16 * gi, kVec, t);
#pragma unroll
            for (int q = 0; q < 16; ++q) m = fmaxf(m, fabsf(t[q]));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    if (!active) return;
    const int e = column_exponent(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
    if (tid == 0) xe[n] = e;
    if (resident) {
#pragma unroll
        for (int u = 0; u < kPreGroups; ++u) {
            const int gi = tid + 256 * u;
            if (gi < groups) store16_perm<HL>(v[u], e, x16 + n * K + 16 * gi, lo_off);
        }
    } else {
        for (int gi = tid; gi < groups; gi += 256) {
            float t[16];
            load16(col + 16 * gi, kVec, t);
            store16_perm<HL>(t, e, x16 + n * K + 16 * gi, lo_off);
        }
    }
}

}  // namespace q2_0
