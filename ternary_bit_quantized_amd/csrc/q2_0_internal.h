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
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// IEEE half bits -> f32 (v_cvt_f32_f16: exact for every half, subnormals included).
__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// ---- activation element types (Q2_0_ACT_*).  Every kernel reads activations through
// these helpers and computes on the exact f32 value of each element.
enum class Act { F32 = Q2_0_ACT_F32, F16 = Q2_0_ACT_F16, BF16 = Q2_0_ACT_BF16 };

struct bf16_t {   // bfloat16: the upper 16 bits of an IEEE single
    uint16_t bits;
};

inline int act_bytes(Act a) { return a == Act::F32 ? 4 : 2; }

__device__ __forceinline__ float act_to_f32(float v) { return v; }
__device__ __forceinline__ float act_to_f32(_Float16 v) { return (float)v; }
__device__ __forceinline__ float act_to_f32(bf16_t v) { return __builtin_bit_cast(float, (uint32_t)v.bits << 16); }

// Four consecutive activations as f32; p is aligned to four elements (16 bytes for
// f32, 8 bytes for the 16-bit types).
template <typename XT>
__device__ __forceinline__ float4_t load_act4(const XT *p);

template <>
__device__ __forceinline__ float4_t load_act4<float>(const float *p) {
    return *reinterpret_cast<const float4_t *>(p);
}

template <>
__device__ __forceinline__ float4_t load_act4<_Float16>(const _Float16 *p) {
    typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
    const half4_t v = *reinterpret_cast<const half4_t *>(p);
    return float4_t{(float)v.x, (float)v.y, (float)v.z, (float)v.w};
}

template <>
__device__ __forceinline__ float4_t load_act4<bf16_t>(const bf16_t *p) {
    const u32x2_t v = *reinterpret_cast<const u32x2_t *>(p);
    return float4_t{__builtin_bit_cast(float, v.x << 16), __builtin_bit_cast(float, v.x & 0xffff0000u),
                    __builtin_bit_cast(float, v.y << 16), __builtin_bit_cast(float, v.y & 0xffff0000u)};
}

// Two consecutive activations as f32; p is aligned to two elements.
template <typename XT>
__device__ __forceinline__ float2_t load_act2(const XT *p);

template <>
__device__ __forceinline__ float2_t load_act2<float>(const float *p) {
    return *reinterpret_cast<const float2_t *>(p);
}

template <>
__device__ __forceinline__ float2_t load_act2<_Float16>(const _Float16 *p) {
    const half2_t v = *reinterpret_cast<const half2_t *>(p);
    return float2_t{(float)v.x, (float)v.y};
}

template <>
__device__ __forceinline__ float2_t load_act2<bf16_t>(const bf16_t *p) {
    const uint32_t v = *reinterpret_cast<const uint32_t *>(p);
    return float2_t{__builtin_bit_cast(float, v << 16), __builtin_bit_cast(float, v & 0xffff0000u)};
}

// Runs f(XT{}) with XT the element type of a (host side).
template <typename F>
inline hipError_t with_act(Act a, F &&f) {
    switch (a) {
        case Act::F32: return f(float{});
        case Act::F16: return f(_Float16{});
        case Act::BF16: return f(bf16_t{});
    }
    return hipErrorInvalidValue;
}

// Scale and one 32-bit code word of block `blk` from a 2-byte aligned block base.
// Word w sits at byte 2 + 4w: 4-byte aligned only for odd blocks of an aligned row,
// so it is read as two half-words.
__device__ __forceinline__ uint32_t load_word_u16x2(const uint16_t *blk16, int w) {
    return (uint32_t)blk16[1 + 2 * w] | ((uint32_t)blk16[2 + 2 * w] << 16);
}

// Argument checks of q2_0_mul_mat other than the workspace (api.hip); *noop is set
// for the empty no-op.  record_hip_error stores e as the calling thread's last HIP error
// and returns the status for it.
int check_mul_mat(const void *w, int64_t M, int64_t K, const void *x, int x_type, int64_t ldx, int64_t N,
                  const float *y, int64_t ldy, int precision, bool *noop);
int record_hip_error(hipError_t e);

// Launchers (return the HIP error of the launch).
hipError_t launch_get_rows(const uint8_t *w, int64_t M, int nb, const int32_t *ids, int64_t n_ids,
                           float *out, int64_t ld_out, hipStream_t s);
// x points at activations of element type xt; ldx counts elements.
hipError_t launch_mat_vec(const uint8_t *w, int64_t M, int nb, const void *x, Act xt, int64_t ldx, int N,
                          float *y, int64_t ldy, hipStream_t s);
// the generic f32 kernel only (no condition on the activations' range)
hipError_t launch_mat_vec_f32(const uint8_t *w, int64_t M, int nb, const void *x, Act xt, int64_t ldx, int N,
                              float *y, int64_t ldy, hipStream_t s);
hipError_t launch_mat_vec_group(const q2_0_mat_vec_item *items, int64_t n_items, int nb,
                                const void *x, Act xt, int64_t ldx, int N, hipStream_t s);
hipError_t launch_mat_vec_batch(const q2_0_mat_vec_batch_item *items, int64_t n_items, Act xt, int N,
                                hipStream_t s);
bool mat_vec_mfma_eligible(const uint8_t *w, int64_t M, int nb, const void *x, Act xt, int64_t ldx);
hipError_t launch_mat_vec_mfma(const uint8_t *w, int64_t M, int nb, const void *x, Act xt, int64_t ldx,
                               int N, float *y, int64_t ldy, hipStream_t s);
// fp16-MFMA GEMM over one or more matrices that share K and x (items: w, M, y, ldy).
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
    // Expert routing (mul_mat_id), when moe_off is set: workgroup b takes row tile
    // b % moe_tiles_m of the (expert, column tile) entry b / moe_tiles_m of moe_tiles
    // (device; *moe_ntiles entries, the rest exit); expert e is the matrix at
    // p[0].w + e * moe_expert_bytes, its columns are x16 columns moe_off[e] ..
    // moe_off[e+1]-1, and result column j goes to y column moe_perm[j] of p[0]; it
    // multiplies x16 row moe_perm[j] / moe_xdiv (the token's x row, shared by its slots
    // when moe_xdiv is the slots per token).
    const int *moe_off;
    const int *moe_perm;
    const int *moe_tiles;     // pairs (expert, column tile)
    const int *moe_ntiles;
    int64_t moe_expert_bytes;
    int moe_tiles_m;
    int moe_xdiv;
    // the tile list's bound: workgroups past moe_max_tiles * moe_tiles_m fill the y
    // columns of the out-of-range run (moe_off[moe_n_expert] ..) with NaN, one row tile each
    int moe_max_tiles;
    int moe_n_expert;
};
// hl: x as fp16 hi/lo pairs, per-block sums added in fp64 (the fp32-grade GEMM)
size_t gemm_f16_workspace_bytes(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K, int64_t N,
                                bool hl = false);
// the K split the call's plan picks (1: none)
int gemm_f16_splits(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K, int64_t N, bool hl = false);
hipError_t launch_gemm_f16_group(const q2_0_mat_vec_item *items, int64_t n_items, int nb, const void *x, Act xt,
                                 int64_t ldx, int64_t N, void *workspace, hipStream_t s, bool hl = false);
hipError_t launch_gemm_f32(const uint8_t *w, int64_t M, int nb, const void *x, Act xt, int64_t ldx,
                           int64_t N, float *y, int64_t ldy, hipStream_t s);

// ---- expert product (mul_mat_id).  Routing tables in device memory: off[e] .. off[e+1]
// are the sorted positions of expert e's (token, slot) pairs (e = n_expert: ids out of
// range), perm[j] the pair at sorted position j (pair p = t * n_used + u).
// tiles: (expert, column tile of tile_w columns) for every tile an expert has, in expert
// order, *ntiles of them (at most moe_max_tiles()).
struct MoeRoute {
    const int *off;       // n_expert + 2 entries
    const int *perm;      // n_pairs entries
    const int *tiles;     // 2 * moe_max_tiles() entries
    const int *ntiles;
    int n_expert;
    int n_pairs;
    int n_used;
    int x_slots;          // 1: every slot of a token uses x column t; n_used: column t*n_used + u
    int tile_w;
};
inline int64_t moe_max_tiles(int64_t n_expert, int64_t n_pairs, int tile_w) {
    return (n_expert < n_pairs ? n_expert : n_pairs) + (n_pairs + tile_w - 1) / tile_w;
}
size_t moe_route_bytes(int64_t n_expert, int64_t n_pairs, int tile_w);
// Lays out the routing tables in ws (moe_route_bytes bytes) and enqueues the routing.
hipError_t launch_moe_route(const int32_t *ids, int n_pairs, int n_expert, int n_used, int x_slots, int tile_w,
                            void *ws, MoeRoute *r, hipStream_t s);
// x rows of an expert call: one per token (x_slots == 1) or one per pair
inline int moe_x_rows(int n_pairs, int n_used, int x_slots) { return x_slots == 1 ? n_pairs / n_used : n_pairs; }
// The routing and, in the same launch, the fp16 GEMM's x (x16 and its row exponents at
// scratch, laid out as launch_gemm_f16_moe reads them).  Returns false (and launches
// nothing) when the routing takes the kernel for many experts; then launch_moe_route
// and launch_gemm_f16_moe's own conversion do the work.
bool moe_route_converts(int n_expert);
hipError_t launch_moe_route_convert(const int32_t *ids, int n_pairs, int n_expert, int n_used, int x_slots,
                                    int tile_w, void *ws, MoeRoute *r, const void *x, Act xt, int64_t ldx, int K,
                                    void *scratch, hipStream_t s);
// x_ready: x16 and its exponents are already in scratch (launch_moe_route_convert)
hipError_t launch_gemm_f16_moe(const uint8_t *w, int64_t M, int nb, const void *x, Act xt, int64_t ldx,
                               const MoeRoute &r, float *y, int64_t ldy, void *scratch, hipStream_t s,
                               bool x_ready = false);
size_t gemm_f16_moe_scratch_bytes(int64_t K, int64_t n_pairs);
hipError_t launch_moe_fill_bad(const MoeRoute &r, int64_t M, float *y, int64_t ldy, hipStream_t s);
// few tokens: one K-split mat-vec per pair, expert read from ids on the GPU; pairs with
// ids out of range get NaN columns from the same launch
hipError_t launch_mat_vec_mfma_pairs(const uint8_t *w, int64_t M, int nb, const void *x, Act xt, int64_t ldx,
                                     const int32_t *ids, int n_expert, int n_used, int x_slots, int n_pairs,
                                     float *y, int64_t ldy, hipStream_t s);
hipError_t launch_gemm_f32_moe(const uint8_t *w, int64_t M, int nb, const void *x, Act xt, int64_t ldx,
                               const MoeRoute &r, float *y, int64_t ldy, hipStream_t s);

hipError_t launch_quantize(const float *src, int64_t M, int nb, int64_t ld, uint8_t *w, hipStream_t s);
hipError_t launch_repack_g128(const uint8_t *w128, int64_t M, int64_t K, uint8_t *w, hipStream_t s);

}  // namespace q2_0
