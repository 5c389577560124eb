// Device building blocks shared by the MFMA mat-vec kernels (gfx950).
//
// Arithmetic (bisque.today "WebGPU: add Q2_0 support", the matrix-vector
// paragraph): each 64-weight block contributes d * sum (q - 1) * x, the scale
// applied once to the block's sum.  On gfx950 the block sum runs on the matrix
// cores: v_mfma_f32_16x16x32_f16 with the activation as the A operand (A row 2n =
// fp16(x_n), row 2n+1 = fp16(x_n - fp16(x_n)), so hi + lo carries ~22 bits of x)
// and the exact fp16 values q - 1 as B (16 weight rows as the 16 B columns).  D
// lane (j, g) then holds, for weight row j, x rows 4g..4g+3 = columns 2g and 2g+1
// as (hi, lo) pairs.
//
// Weight layout in the wave's LDS tile: rows are 16-byte aligned, so a block pair
// is 9 dwords D0..D8: D0 = [d_b | h0], D1..D3 = [h1|h2] [h3|h4] [h5|h6], D4 =
// [h7 | d_b+1], D5..D8 = [h0|h1] .. [h6|h7] of block b+1 (h_i = the 8 codes of
// weights 8i..8i+7).  Lane group g takes one code dword per block: even blocks
// (h0,h7) (h1,h2) (h3,h4) (h5,h6), odd blocks (h0,h1) .. (h6,h7).  The A operand
// is staged in the same pairing, so B element 2e+h multiplies the x of the same
// weight.
#pragma once

#include <cstddef>

#include "q2_0_internal.h"

namespace q2_0 {

constexpr int kMvTile = 16;        // weight rows per MFMA tile
constexpr int kMvStreamSB = 16;    // blocks per stage in the streaming kernel
constexpr int kMvMaxGroup = 64;    // matrices per grouped launch (kernel argument size)
constexpr size_t kMvStreamStaticLds = 1024;  // static LDS bound of the streaming kernel
constexpr int kMvStreamMaxWaves = 16;        // largest streaming workgroup (waves)
constexpr int kMvBcastRows = 16;             // rows per tile of the broadcast kernel

struct MvProblem {
    const uint8_t *w;
    float *y;
    int64_t ldy;
    int M;
    int tile0;   // first tile number of this matrix within the group
};

// A launch's matrices.  tile0 repeats the problems' first tiles contiguously (entries
// from n on, including the extra last one, hold INT_MAX), so that a tile's matrix is
// found by a binary search of log2(kMvMaxGroup) scalar loads, and tile0[i + 1] bounds
// matrix i.
struct MvGroup {
    MvProblem p[kMvMaxGroup];
    int tile0[kMvMaxGroup + 1];
    int n;
    int total_tiles;
};

// The launch's tile table, one entry per lane: lane i holds grp.tile0[i] (i < 64;
// entries from n on are INT_MAX).  Loaded once per wave with one vector load from the
// kernel arguments, it turns every later matrix lookup into a ballot.
__device__ __forceinline__ int load_tile_table(const MvGroup &grp) {
    static_assert(kMvMaxGroup == 64, "one table entry per lane");
    // (a C cast: the kernel-argument address space converts to a generic pointer)
    const int *t = (const int *)((const uint8_t *)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(MvGroup, tile0));
    return t[__lane_id()];
}

// The last i with tile0[i] <= tile (tile0 ascends, so those i are a prefix); uniform.
__device__ __forceinline__ int find_problem(int t0v, int tile) {
    return (int)__popcll(__ballot(t0v <= tile)) - 1;
}

// The wave's current matrix and tile, all wave-uniform.
struct TileRef {
    const uint8_t *w;
    float *y;
    int64_t ldy;
    int M;
    int m0;
};

template <int TILE>
__device__ __forceinline__ TileRef tile_ref(const MvGroup &grp, int t0v, int tile) {
    const int idx = find_problem(t0v, tile);
    const MvProblem &p = grp.p[idx];
    return TileRef{p.w, p.y, p.ldy, p.M, (tile - __builtin_amdgcn_readlane(t0v, idx)) * TILE};
}

// A wave's tiles only move forward, so it follows them with a cursor: the current
// matrix's fields and tile range stay in SGPRs, and the kernel arguments are read again
// only when a tile passes the end of that matrix.
struct TileCursor {
    TileRef r;   // r.m0 is that of the matrix's first tile (0)
    int idx, t0, t1;
};

__device__ __forceinline__ void cursor_load(const MvGroup &grp, int t0v, TileCursor &c) {
    const MvProblem &p = grp.p[c.idx];
    c.r = TileRef{p.w, p.y, p.ldy, p.M, 0};
    c.t0 = __builtin_amdgcn_readlane(t0v, c.idx);
    c.t1 = c.idx + 1 < kMvMaxGroup ? __builtin_amdgcn_readlane(t0v, c.idx + 1) : 0x7fffffff;
}

__device__ __forceinline__ void cursor_init(const MvGroup &grp, int t0v, TileCursor &c, int tile) {
    c.idx = find_problem(t0v, tile);
    cursor_load(grp, t0v, c);
}

// The tile's matrix and rows (TILE rows per tile).  Tiles mostly move forward; a tile
// outside the cursor's matrix (past it, or before it when a wave starts the next
// window of its tiles) looks the matrix up again.
template <int TILE>
__device__ __forceinline__ TileRef cursor_tile(const MvGroup &grp, int t0v, TileCursor &c, int tile) {
    if (tile >= c.t1 || tile < c.t0) {
        c.idx = find_problem(t0v, tile);
        cursor_load(grp, t0v, c);
        // wait for the argument loads here, on the rare path: a wait left to the join
        // would also wait, on every tile, for the LDS stores just issued (one counter
        // covers both).  lgkmcnt(0), vmcnt and expcnt untouched.
        __builtin_amdgcn_s_waitcnt(0xc07f);
    }
    TileRef t = c.r;
    t.m0 = (tile - c.t0) * TILE;
    return t;
}

// floor(a * b / c) for 0 <= a, b and 0 < c with a * b < 2^53, without a 64-bit integer
// division: the double quotient, corrected by at most one either way.
__device__ __forceinline__ int64_t mul_div(int64_t a, int64_t b, int64_t c) {
    const int64_t p = a * b;
    int64_t q = (int64_t)((double)p / (double)c);
    if (q * c > p) --q;
    else if ((q + 1) * c <= p) ++q;
    return q;
}

__device__ __forceinline__ int64_t div_floor(int64_t a, int64_t c) { return mul_div(a, 1, c); }

__device__ __forceinline__ half8_t as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(half8_t, u4{a, b, c, d});
}

// (a & mask) | orv as one v_and_or_b32.  gfx9 VOP3 encodings take no literal and
// read at most one SGPR, so the mask must sit in a VGPR for the compiler to select
// the fused form; otherwise it splits the expression into a v_and and a v_or.
// The masks are therefore materialised once through an opaque v_mov (which keeps
// the compiler from folding them back into literals), and the AND-OR itself is
// plain code, so the compiler's own hazard tracking covers it (it does not see
// into inline asm, which matters next to MFMAs writing VGPRs).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t orv) {
    return (a & mask) | orv;
}

// Masks selecting code s (s = 0..4) of both 16-bit halves, held in VGPRs.
struct PairMasks {
    uint32_t m[5];
    __device__ __forceinline__ PairMasks() {
        asm volatile("v_mov_b32 %0, 0x30003" : "=v"(m[0]));
        asm volatile("v_mov_b32 %0, 0xc000c" : "=v"(m[1]));
        asm volatile("v_mov_b32 %0, 0x300030" : "=v"(m[2]));
        asm volatile("v_mov_b32 %0, 0xc000c0" : "=v"(m[3]));
        asm volatile("v_mov_b32 %0, 0x3000300" : "=v"(m[4]));
    }
};

// fp16 pair (q_s - 1 of the low half, q_s - 1 of the high half) of a code dword, for
// codes at mantissa bits 2s, 2s+1 (s = 0..4).  OR-ing the code under the exponent
// 25 - 2s gives the half 2^(10-2s) + q exactly; subtracting 2^(10-2s) + 1 leaves
// q - 1 exactly.
template <int S>
__device__ __forceinline__ uint32_t pair_qm1(uint32_t cd, const PairMasks &pm) {
    constexpr uint32_t magic = (uint32_t)(25 - 2 * S) << 10;
    constexpr float off = (float)((1 << (10 - 2 * S)) + 1);
    const uint32_t t = and_or(cd, pm.m[S], magic | (magic << 16));
    half2_t h = __builtin_bit_cast(half2_t, t);
    h = h - half2_t{(_Float16)off, (_Float16)off};
    return __builtin_bit_cast(uint32_t, h);
}

// The 8 pairs of a code dword: pairs 0..3 feed the block's first MFMA, 4..7 the
// second.  Pair s takes code s of both halves.
__device__ __forceinline__ void decode_dword(uint32_t cd, const PairMasks &pm, half8_t &b0,
                                             half8_t &b1) {
    const uint32_t hi = cd >> 10;   // codes 5..7 of each half down to bits 0..5
    b0 = as_half8(pair_qm1<0>(cd, pm), pair_qm1<1>(cd, pm), pair_qm1<2>(cd, pm), pair_qm1<3>(cd, pm));
    b1 = as_half8(pair_qm1<4>(cd, pm), pair_qm1<0>(hi, pm), pair_qm1<1>(hi, pm), pair_qm1<2>(hi, pm));
}

__device__ __forceinline__ int half_lo(int g, int odd) { return odd ? 2 * g : (g == 0 ? 0 : 2 * g - 1); }
__device__ __forceinline__ int half_hi(int g, int odd) { return odd ? 2 * g + 1 : (g == 0 ? 7 : 2 * g); }

// Activation range.  fp16 holds x to ~22 bits as hi + lo only for |x| in about
// [2^-3, 2^15]: above 65504 hi overflows, and below 2^-3 lo loses bits to fp16's
// subnormal spacing (2^-24).  Each column n is therefore staged as x * 2^e_n, with
// the power of two chosen so that the column's max |x| lands in [2^14, 2^15), and
// its results are multiplied by 2^-e_n on the way out (v_ldexp_f32 both times, exact
// barring f32 under/overflow).  Elements within 2^17 of the column maximum keep
// 2^-22 relative accuracy; smaller ones err by at most 2^-39 of the maximum.
// An all-zero (or non-finite) maximum keeps e = 0.
// TOP: the staged maximum lies in [2^(TOP-1), 2^TOP).
template <int TOP = 15>
__device__ __forceinline__ int column_exponent(float amax) {
    if (!(amax > 0.f) || amax > 3.4028234663852886e38f) return 0;
    return TOP - __builtin_amdgcn_frexp_expf(amax);
}

__device__ __forceinline__ float max_abs4(float4_t v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// Column exponents of x (NC columns of K activations of type XT, aligned to four
// elements, ldx % 4 == 0) into lds_e[0..NC), computed by the whole workgroup; lds_tmp
// holds NC floats per wave.  Each pass issues up to 8 independent 4-element loads per
// thread before reducing, so the scan costs about one memory latency per pass.
// Contains two workgroup barriers, so every thread must call it.
template <int NC, int TOP = 15, typename XT = float>
__device__ __forceinline__ void column_exponents(const XT *__restrict__ x, int64_t ldx, int K,
                                                 int *lds_e, float *lds_tmp, int tid, int nthreads) {
    constexpr int U = (NC >= 8) ? 1 : 8 / NC;   // loads per column per pass
    const int k4 = K / 4;
    float m[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) m[n] = 0.f;
    for (int base = tid; base < k4; base += U * nthreads) {
        float4_t v[NC][U];
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const XT *xc = x + n * ldx;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = base + u * nthreads;
                v[n][u] = (i < k4) ? load_act4(xc + 4 * i) : float4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int n = 0; n < NC; ++n)
#pragma unroll
            for (int u = 0; u < U; ++u) m[n] = fmaxf(m[n], max_abs4(v[n][u]));
    }
#pragma unroll
    for (int n = 0; n < NC; ++n)
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m[n] = fmaxf(m[n], __shfl_xor(m[n], off));
    const int wave = tid >> 6;
    if ((tid & 63) == 0) {
#pragma unroll
        for (int n = 0; n < NC; ++n) lds_tmp[wave * NC + n] = m[n];
    }
    __syncthreads();
    if (tid < NC) {
        float a = 0.f;
        for (int wv = 0; wv < nthreads / 64; ++wv) a = fmaxf(a, lds_tmp[wv * NC + tid]);
        lds_e[tid] = column_exponent<TOP>(a);
    }
    __syncthreads();
}

// One A-operand item: column n, lane group gg, MFMA mu of block blk.  Loaded as the
// two runs of 4 consecutive x the item pairs, then written as two LDS entries (hi
// row 2n, lo row 2n+1) of 8 halves each.
struct XItem {
    float4_t a, c;
};

template <typename XT>
__device__ __forceinline__ XItem load_x_item(const XT *__restrict__ x, int64_t ldx, int blk, int mu,
                                             int gg, int n) {
    const int odd = blk & 1;
    const XT *xb = x + n * ldx + (int64_t)blk * kBlockWeights + 4 * mu;
    return XItem{load_act4(xb + 8 * half_lo(gg, odd)), load_act4(xb + 8 * half_hi(gg, odd))};
}

// xe: the column's exponent (x is staged as x * 2^xe).
__device__ __forceinline__ void store_x_item(const XItem &it, int xe, half8_t *dst) {
    uint32_t hiw[4], low[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float va = __builtin_amdgcn_ldexpf(it.a[e], xe), vc = __builtin_amdgcn_ldexpf(it.c[e], xe);
        const _Float16 ha = (_Float16)va, hc = (_Float16)vc;
        const _Float16 la = (_Float16)(va - (float)ha), lc = (_Float16)(vc - (float)hc);
        hiw[e] = __builtin_bit_cast(uint32_t, half2_t{ha, hc});
        low[e] = __builtin_bit_cast(uint32_t, half2_t{la, lc});
    }
    dst[0] = as_half8(hiw[0], hiw[1], hiw[2], hiw[3]);
    dst[1] = as_half8(low[0], low[1], low[2], low[3]);
}

// Stage x for blocks 0..nb-1: entry ((b*2 + mu)*4 + g)*2NC + row; lds_e holds the
// column exponents.
template <int NC, typename XT>
__device__ __forceinline__ void stage_x_all(const XT *__restrict__ x, int64_t ldx, int nb,
                                            const int *lds_e, half8_t *lds_x, int tid, int nthreads) {
    const int items = nb * 2 * 4 * NC;
    for (int q = tid; q < items; q += nthreads) {
        const int n = q % NC, gg = (q / NC) % 4, mu = (q / (4 * NC)) % 2, b = q / (8 * NC);
        store_x_item(load_x_item(x, ldx, b, mu, gg, n), lds_e[n], lds_x + (q / NC) * (2 * NC) + 2 * n);
    }
}

// One block pair: lp points at the pair's 36 bytes of this lane's row in LDS, a at
// the A entry of (even block, mu = 0) for this lane; entries of (block, mu) are
// 4*2NC apart.  acc0/acc1 accumulate even/odd blocks for columns 2g, 2g+1.
template <int NC>
__device__ __forceinline__ void mv_block_pair(const uint8_t *lp, const half8_t *a, int g, uint32_t sel,
                                              const PairMasks &pm, float acc0[2], float acc1[2]) {
    constexpr int NR = 2 * NC;
    const uint32_t X = *reinterpret_cast<const uint32_t *>(lp + 4 * g);
    const uint32_t Y = *reinterpret_cast<const uint32_t *>(lp + 16);
    const uint32_t Z = *reinterpret_cast<const uint32_t *>(lp + 20 + 4 * g);
    uint32_t D0 = X;   // group 0 reads D0 anyway; only columns of group 0 exist for NC <= 2
    if (NC > 2) D0 = *reinterpret_cast<const uint32_t *>(lp);
    // even block: group 0 pairs h0 (high half of D0) with h7 (low half of D4)
    const uint32_t cde = __builtin_amdgcn_perm(Y, X, sel);
    half8_t b0, b1, c0, c1;
    decode_dword(cde, pm, b0, b1);
    decode_dword(Z, pm, c0, c1);
    float4_t ce = {0.f, 0.f, 0.f, 0.f}, co = {0.f, 0.f, 0.f, 0.f};
    ce = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], b0, ce, 0, 0, 0);
    ce = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[4 * NR], b1, ce, 0, 0, 0);
    co = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[8 * NR], c0, co, 0, 0, 0);
    co = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[12 * NR], c1, co, 0, 0, 0);
    const float de = half_bits_to_float(D0 & 0xffffu);
    const float dd = half_bits_to_float(Y >> 16);
    acc0[0] = __builtin_fmaf(de, ce[0] + ce[1], acc0[0]);
    acc1[0] = __builtin_fmaf(dd, co[0] + co[1], acc1[0]);
    if (NC > 1) {
        acc0[1] = __builtin_fmaf(de, ce[2] + ce[3], acc0[1]);
        acc1[1] = __builtin_fmaf(dd, co[2] + co[3], acc1[1]);
    }
}

// ---- segments of a broadcast-kernel launch: runs of the group's tiles that share one
// activation.  The host describes them (MvSegDesc); the launch adds its own layout
// (MvSeg: the window of stages staged at a time, the segment's workgroups).
constexpr int kMvMaxSegs = 8;
struct MvSegDesc {
    const void *x;    // activations of the launch's element type, column n at x + n*ldx
    int64_t ldx;
    int nb;           // blocks per row (K / 64)
    int tile0, tile1; // the segment's tiles, numbered across the group
};
struct MvSeg {
    const void *x;
    int64_t ldx;
    int nb;
    int ws;           // stages per window: the activation is staged ws*16 blocks at a time
    int tile0, tile1;
    int wg0, wgs;     // the segment's workgroups
    int q, r;         // tiles per workgroup: q, and one more for the first r workgroups
    uint32_t mag_w, mag_last;   // ceil(2^32 / d) for d = the stages of a window, of the last window
};
struct MvSegs {
    MvSeg s[kMvMaxSegs];
    int n;
    int xcap;         // blocks of activation staged in LDS (the largest window)
    int tacc;         // tiles per workgroup of the result accumulator (segments of several windows)
};

size_t mat_vec_stream_lds(int N, int nb, int waves);
int mat_vec_stream_waves(int N, int nb, int *resident);
// rowstride: bytes between rows (0: nb * 18); accumulate: add to y instead of writing it
hipError_t launch_mat_vec_stream(const MvGroup &grp, int nb, const void *x, Act xt, int64_t ldx, int N,
                                 hipStream_t s, uint32_t rowstride = 0, int accumulate = 0);
// N >= 3, any K: one launch where the whole activation fits in LDS, else consecutive launches
// over chunks of mat_vec_stream_chunk_blocks(N, nb) blocks (0: not even one stage fits)
int mat_vec_stream_chunk_blocks(int N, int nb);
hipError_t launch_mat_vec_stream_chunked(const MvGroup &grp, int nb, const void *x, Act xt, int64_t ldx, int N,
                                         hipStream_t s);
// N = 1, 2; grp counts tiles of kMvBcastRows rows; nsegs <= kMvMaxSegs segments.  Any K
// (the activation is staged in windows); rows and activations 16-byte aligned, nb % 8 == 0.
size_t mat_vec_bcast_lds(int N, int xcap, int tacc, int waves, bool exact);
hipError_t launch_mat_vec_bcast(const MvGroup &grp, const MvSegDesc *segs, int nsegs, Act xt, int N,
                                hipStream_t s);

}  // namespace q2_0
