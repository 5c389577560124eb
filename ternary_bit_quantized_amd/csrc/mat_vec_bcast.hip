// Persistent mat-vec for N = 1, 2 on the gfx950 matrix cores' 16-block 4x4x4
// product, with the activation broadcast from registers inside groups of 16 lanes.
//
// Arithmetic (bisque.today "WebGPU: add Q2_0 support", the matrix-vector paragraph: per
// 64-weight block the sum of (q - 1) * x, multiplied by the block scale once), in one of
// two modes, products exact either way:
//  * exact mode (N = 1): each block of x as four 11-bit fixed-point limbs, the codes
//    raw; every block sum is exact (described at bx_dword below);
//  * hi/lo mode (N = 2): exact fp16 (q - 1) from the pair decode against x as an fp16
//    hi/lo pair, each column scaled by a power of two; sums in f32.
//
// The product: v_mfma_f32_4x4x4_16b_f16 runs 16 independent 4x4x4 products, block b
// on lanes 4b..4b+3; with CBSZ = 2 the blocks form 4 groups of 4 (16 lanes each), and
// every block of group G takes the A operand of block 4G + ABID.  Lane 16G + 4a + i
// holds A row i of chunk a, a chunk being 4 activations, the rows limbs 0..3 (exact
// mode) or column 0 hi, lo and column 1 hi, lo (hi/lo mode).  One pair of VGPRs thus
// holds, for each group, the 16 activations of one code dword, and ABID = 0..3 on 4
// successive products selects its chunks.  B column 16G + r is weight row r of the
// tile, i.e. the lane: group G's lanes decode the 16 rows' blocks of quarter G of the
// stage, and each lane accumulates its own (row, quarter) sum in D items 0..3.  The
// four quarters of a row are added once per tile by two lane exchanges.  Activation
// reads from LDS: one 8-byte read per code dword and lane, a quarter of what the
// 16x16x32 form needs.
//
// Streaming as in mat_vec_stream.hip: work items (16-row tile, stage of 16 blocks),
// tile-major, split evenly over persistent workgroups and their waves; each wave keeps
// one stage in flight in registers -- coalesced 16-byte loads, consecutive lanes on consecutive
// bytes of a row: 16 rows x 288 bytes, a pattern that reads at ~96 % of a contiguous
// stream's rate -- while it decodes the previous one from a wave-private LDS tile.
// The park routes each 8-byte half of a loaded chunk to the LDS area of its quarter (80
// bytes per quarter, 16-byte aligned), from which each lane reads its quarter with five
// 16-byte reads.  The activation is staged in windows of whole stages (phases); a tile
// whose stages are split between waves is finished after the phase's barrier, in stage
// order, so results are deterministic.
#include <algorithm>
#include <atomic>

#include "q2_0_internal.h"
#include "mat_vec_common.h"

namespace q2_0 {

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

constexpr int kBcRows = kMvBcastRows;                  // weight rows per tile
constexpr int kBcSB = 16;                              // blocks per stage: 4 per quarter
constexpr int kBcCPR = kBcSB * kBlockBytes / 16;       // 16-byte chunks per row and stage (18)
constexpr int kBcNCH = kBcRows * kBcCPR;               // chunks per stage (288)
constexpr int kBcCH = (kBcNCH + 63) / 64;              // chunks per lane (5; the last round part empty)
constexpr int kBcQuarter = 80;                         // LDS bytes per (row, quarter): 72 used
// LDS row stride: 4 quarters, padded so that the 8 lanes of one 16-byte read phase
// (rows r..r+7 of one quarter) fall on distinct banks (84 dwords: 20 apart mod 32)
constexpr int kBcRS = 4 * kBcQuarter + 16;
constexpr int kBcWaveLds = kBcRows * kBcRS;            // a wave's weight tile in LDS
static_assert(kBcRS % 16 == 0 && kBcSB * kBlockBytes == 4 * 72, "stage geometry");

struct BcItem {
    int tile, st;
};

typedef uint32_t u32x2a8_t __attribute__((ext_vector_type(2), aligned(8)));

__device__ __forceinline__ half4_t as_half4(uint32_t a, uint32_t b) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(half4_t, u2{a, b});
}

// Chunk A of the lane group's current code dword times the decoded B.
template <int A>
__device__ __forceinline__ float4_t bc_mfma(half4_t xa, half4_t b, float4_t acc) {
    return __builtin_amdgcn_mfma_f32_4x4x4f16(xa, b, acc, 2, A, 0);
}

// One code dword with half-words (h_A, h_B): chunk t takes the decode pairs 2t and
// 2t+1, i.e. the block's weights 8A+2t, 8B+2t, 8A+2t+1, 8B+2t+1; xa holds the group's
// activations of those 16 weights in that order.
__device__ __forceinline__ float4_t bc_dword(uint32_t cd, half4_t xa, const PairMasks &pm, float4_t acc) {
    const uint32_t hi = cd >> 10;   // codes 5..7 of each half down to bits 0..5
    acc = bc_mfma<0>(xa, as_half4(pair_qm1<0>(cd, pm), pair_qm1<1>(cd, pm)), acc);
    acc = bc_mfma<1>(xa, as_half4(pair_qm1<2>(cd, pm), pair_qm1<3>(cd, pm)), acc);
    acc = bc_mfma<2>(xa, as_half4(pair_qm1<4>(cd, pm), pair_qm1<0>(hi, pm)), acc);
    acc = bc_mfma<3>(xa, as_half4(pair_qm1<1>(hi, pm), pair_qm1<2>(hi, pm)), acc);
    return acc;
}

// This lane's row over one block: item r = sum of (q - 1) times A row r.
__device__ __forceinline__ float4_t bc_block(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                             const half4_t *xa, const PairMasks &pm) {
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    acc = bc_dword(c0, xa[0], pm, acc);
    acc = bc_dword(c1, xa[1], pm, acc);
    acc = bc_dword(c2, xa[2], pm, acc);
    acc = bc_dword(c3, xa[3], pm, acc);
    return acc;
}

// This lane's quarter of a stage (4 blocks = two block pairs) of its row.  R: the 72
// bytes, as dwords 0..17.  A pair is 9 dwords D0..D8 (layout in mat_vec_common.h): the
// even block's scale is the low half of D0 and its code dwords (h0,h7) (h1,h2) (h3,h4)
// (h5,h6), the odd block's scale the high half of D4 and its code dwords D5..D8.
// xs: the lane's A entry of the quarter's first block (entries of block b, code dword u at
// xs[4 (4b + u) 2NC]), read a block at a time next to its products (all 16 held at once
// took 32 registers and made the kernel spill); acc_e / acc_o accumulate even / odd
// blocks; a quarter outside the row (the empty half of a row's last stage when
// K/64 % 16 == 8) leaves them unchanged.
template <int NC>
__device__ __forceinline__ void bc_quarter(const uint32_t (&R)[20], const half4_t *xs, const PairMasks &pm,
                                           bool valid, float (&acc_e)[2], float (&acc_o)[2]) {
    constexpr int NR = 2 * NC;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int o = 9 * p;
        const uint32_t h0h7 = __builtin_amdgcn_perm(R[o + 4], R[o + 0], 0x05040302u);
        half4_t xe[4], xo[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            xe[u] = xs[4 * (8 * p + u) * NR];
            xo[u] = xs[4 * (8 * p + 4 + u) * NR];
        }
        // scheduling fences keep the decode of one block next to its products (hoisted
        // ahead, the decoded halves of several blocks would not fit in registers)
        __builtin_amdgcn_sched_barrier(0);
        const float4_t se = bc_block(h0h7, R[o + 1], R[o + 2], R[o + 3], xe, pm);
        __builtin_amdgcn_sched_barrier(0);
        const float4_t so = bc_block(R[o + 5], R[o + 6], R[o + 7], R[o + 8], xo, pm);
        __builtin_amdgcn_sched_barrier(0);
        const float de = half_bits_to_float(R[o + 0] & 0xffffu);
        const float dd = half_bits_to_float(R[o + 4] >> 16);
        const float e0 = __builtin_fmaf(de, se[0] + se[1], acc_e[0]);
        const float o0 = __builtin_fmaf(dd, so[0] + so[1], acc_o[0]);
        acc_e[0] = valid ? e0 : acc_e[0];
        acc_o[0] = valid ? o0 : acc_o[0];
        if (NC > 1) {
            const float e1 = __builtin_fmaf(de, se[2] + se[3], acc_e[1]);
            const float o1 = __builtin_fmaf(dd, so[2] + so[3], acc_o[1]);
            acc_e[1] = valid ? e1 : acc_e[1];
            acc_o[1] = valid ? o1 : acc_o[1];
        }
    }
}

// Stage x for blocks 0..nb-1 as the broadcast A operand: entry (blk*16 + c)*2NC + r is
// half4 row r of chunk c = 4u + t of block blk (rows 2n, 2n+1: column n's hi and lo),
// chunk t of code dword u in the weight order of bc_dword.  lds_e holds the column
// exponents.
template <int NC, typename XT>
__device__ __forceinline__ void stage_x_bcast(const XT *__restrict__ x, int64_t ldx, int nb, const int *lds_e,
                                              half4_t *lds_x, int tid, int nthreads) {
    constexpr int NR = 2 * NC;
    constexpr int U = 2;   // items per thread whose loads are issued before any is converted
    const int items = nb * 16 * NC;
    for (int q0 = tid; q0 < items; q0 += U * nthreads) {
        float2_t a[U], b[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int q = min(q0 + k * nthreads, items - 1);
            const int n = q % NC, c = (q / NC) % 16, blk = q / (16 * NC);
            const int u = c >> 2, t = c & 3, odd = blk & 1;
            const XT *xb = x + n * ldx + (int64_t)blk * kBlockWeights + 2 * t;
            a[k] = load_act2(xb + 8 * half_lo(u, odd));
            b[k] = load_act2(xb + 8 * half_hi(u, odd));
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int q = q0 + k * nthreads;
            if (q >= items) break;
            const int n = q % NC, c = (q / NC) % 16, blk = q / (16 * NC);
            const int xe = lds_e[n];
            const float v[4] = {__builtin_amdgcn_ldexpf(a[k].x, xe), __builtin_amdgcn_ldexpf(b[k].x, xe),
                                __builtin_amdgcn_ldexpf(a[k].y, xe), __builtin_amdgcn_ldexpf(b[k].y, xe)};
            half4_t hi, lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hi[e] = (_Float16)v[e];
                lo[e] = (_Float16)(v[e] - (float)hi[e]);
            }
            half4_t *dst = lds_x + (blk * 16 + c) * NR + 2 * n;
            dst[0] = hi;
            dst[1] = lo;
        }
    }
}

// ---- Exact mode (N = 1).
//
// The activation of each block is scaled by a power of two 2^e that puts its largest
// |x| in [2^10, 2^11), and written as four fixed-point limbs of 11 bits,
// x 2^e = L0 + L1 2^-11 + L2 2^-22 + L3 2^-33 with integer L (|L0| <= 2048, |L1..L3| <=
// 1024): every element within 2^20 of the block's largest is represented exactly (its
// 24 bits fit), smaller ones to 2^-44 of the largest.  A row l of the product is limb
// l.  The codes enter raw: code q at mantissa bits 2s, 2s+1 of a half with a zero
// exponent is the fp16 subnormal q 2^(2s-24), one AND per two weights, and the limb
// meeting it is staged as L 2^(4-2s), so every product is L q 2^-20 exactly.  The
// accumulator starts at -2^-20 sum L over the block (the block's value if every code
// were 1), so after the block's 16 products item l holds 2^-20 sum (q - 1) L exactly:
// every partial sum is a multiple of 2^-20 below 2^24 in magnitude.  A weight of zero
// thus contributes nothing at all, whatever its activation.  The block's value is
// 2^20 (D0 + D1 2^-11 + D2 2^-22 + D3 2^-33) 2^-e, times the block scale.

// Code dword, raw: chunk t takes the pairs 2t, 2t+1 as in bc_dword; pair p holds the
// codes at bits 2p of each half (p <= 4) or, from the dword shifted down by 10, at
// bits 2(p - 5) (p >= 5).
__device__ __forceinline__ float4_t bx_dword(uint32_t cd, half4_t xa, float4_t acc) {
    const uint32_t hi = cd >> 10;
    acc = bc_mfma<0>(xa, as_half4(cd & 0x00030003u, cd & 0x000c000cu), acc);
    acc = bc_mfma<1>(xa, as_half4(cd & 0x00300030u, cd & 0x00c000c0u), acc);
    acc = bc_mfma<2>(xa, as_half4(cd & 0x03000300u, hi & 0x00030003u), acc);
    acc = bc_mfma<3>(xa, as_half4(hi & 0x000c000cu, hi & 0x00300030u), acc);
    return acc;
}

// Bit position / 2 of the code that item k of chunk t meets (see bx_dword), and the
// staging factor 2^(4 - 2s) of the limbs it multiplies.
__device__ __forceinline__ float bx_factor(int t, int k) {
    const int pair = 2 * t + (k >> 1);
    const int s = pair <= 4 ? pair : pair - 5;
    return __builtin_amdgcn_ldexpf(1.f, 4 - 2 * s);
}

// This lane's quarter of a stage in exact mode.  xs: the lane's A entry of the quarter's
// first block (entries of block b, code dword u at xs[(16b + 4u) * 4]); bs / bsc: the
// quarter's first block record (-2^-20 sum L per limb, and 2^(20-e)).
__device__ __forceinline__ void bx_quarter(const uint32_t (&R)[20], const half4_t *xs, const float4_t *bs,
                                           const float *bsc, bool valid, float (&acc_e)[2], float (&acc_o)[2]) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int o = 9 * p;
        const uint32_t h0h7 = __builtin_amdgcn_perm(R[o + 4], R[o + 0], 0x05040302u);
        const uint32_t ce[4] = {h0h7, R[o + 1], R[o + 2], R[o + 3]};
        const uint32_t co[4] = {R[o + 5], R[o + 6], R[o + 7], R[o + 8]};
        float r2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int b = 2 * p + h;
            __builtin_amdgcn_sched_barrier(0);
            float4_t acc = bs[b];
#pragma unroll
            for (int u = 0; u < 4; ++u) acc = bx_dword(h ? co[u] : ce[u], xs[(16 * b + 4 * u) * 4], acc);
            __builtin_amdgcn_sched_barrier(0);
            const float c11 = 4.8828125e-4f;   // 2^-11
            const float v = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(acc[3], c11, acc[2]), c11, acc[1]), c11, acc[0]);
            r2[h] = v * bsc[b];
        }
        const float de = half_bits_to_float(R[o + 0] & 0xffffu);
        const float dd = half_bits_to_float(R[o + 4] >> 16);
        const float e0 = __builtin_fmaf(de, r2[0], acc_e[0]);
        const float o0 = __builtin_fmaf(dd, r2[1], acc_o[0]);
        acc_e[0] = valid ? e0 : acc_e[0];
        acc_o[0] = valid ? o0 : acc_o[0];
    }
}

// Max and sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15), the result in every
// lane of the row: four rotations within the row (row_ror 8, 4, 2, 1), each a VALU
// operation, where lane exchanges through the LDS unit cost ~100 cycles apiece.
template <int N>
__device__ __forceinline__ float row_ror(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x120 + N, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, row_ror<8>(v));
    v = fmaxf(v, row_ror<4>(v));
    v = fmaxf(v, row_ror<2>(v));
    return fmaxf(v, row_ror<1>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += row_ror<8>(v);
    v += row_ror<4>(v);
    v += row_ror<2>(v);
    return v + row_ror<1>(v);
}

// Exact-mode staging of one activation column for blocks 0..nb-1: limb entries
// (blk*16 + c)*4 + l (half4 of chunk c = 4u + t, limb l, in the weight order of
// bx_dword, each element times bx_factor), and per block bs = -2^-20 sum L per limb
// (NaN for limb 0 when the block holds a non-finite activation) and bsc = 2^(20-e).  One
// thread per chunk, in passes of kLimbU * nthreads chunks whose loads are all issued
// before any is converted (limbs_load, then limbs_convert; the kernel issues its first
// weight loads between the two halves of the first pass).  The 16 chunks of a block sit
// in the 16 lanes of a DPP row, which reduce the block's maximum and limb sums (exactly:
// the limbs are integers below 2^12 and a block's sums stay below 2^18, so any order of
// the additions gives the same sum).
constexpr int kLimbU = 2;
struct LimbLoads {
    float2_t a[kLimbU], b[kLimbU];
};

template <typename XT>
__device__ __forceinline__ void limbs_load(const XT *__restrict__ x, int nb, int q0, int tid, int nthreads,
                                           LimbLoads &L) {
    const int items = nb * 16;
#pragma unroll
    for (int k = 0; k < kLimbU; ++k) {
        const int q = min(q0 + k * nthreads + tid, items - 1);
        const int c = q % 16, blk = q / 16;
        const int u = c >> 2, t = c & 3, odd = blk & 1;
        const XT *xb = x + (int64_t)blk * kBlockWeights + 2 * t;
        L.a[k] = load_act2(xb + 8 * half_lo(u, odd));
        L.b[k] = load_act2(xb + 8 * half_hi(u, odd));
    }
}

__device__ __forceinline__ void limbs_convert(int nb, int q0, int tid, int nthreads, const LimbLoads &L,
                                              half4_t *lds_x, float4_t *lds_bs, float *lds_bsc) {
    const int items = nb * 16;
#pragma unroll
    for (int k = 0; k < kLimbU; ++k) {
        if (q0 + k * nthreads >= items) break;      // uniform: whole passes are in or out
        const int q = min(q0 + k * nthreads + tid, items - 1);
        const bool act = q0 + k * nthreads + tid < items;   // whole 16-lane groups are active or not
        const int c = q % 16, blk = q / 16;
        const int t = c & 3;
        const float v[4] = {L.a[k].x, L.b[k].x, L.a[k].y, L.b[k].y};
        const float m = row16_max(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
        const bool finite = m <= 3.4028234663852886e38f;   // false for inf and NaN
        const int e = (finite && m > 0.f) ? 11 - __builtin_amdgcn_frexp_expf(m) : 0;
        float lim[4][4], sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            float w = finite ? __builtin_amdgcn_ldexpf(v[kk], e) : 0.f;
#pragma unroll
            for (int l = 0; l < 4; ++l) {
                const float Lr = __builtin_rintf(w);
                w = (w - Lr) * 2048.f;   // exact: the remainder of a rounded f32 and a power of two
                lim[l][kk] = Lr;
                sum[l] += Lr;
            }
        }
        if (act) {
#pragma unroll
            for (int l = 0; l < 4; ++l) {
                half4_t h;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) h[kk] = (_Float16)(lim[l][kk] * bx_factor(t, kk));
                lds_x[(blk * 16 + c) * 4 + l] = h;
            }
        }
#pragma unroll
        for (int l = 0; l < 4; ++l) sum[l] = row16_sum(sum[l]);
        if (act && c == 0) {
            const float nan = __builtin_nanf("");
            lds_bs[blk] = float4_t{finite ? -sum[0] * 9.5367431640625e-7f : nan, -sum[1] * 9.5367431640625e-7f,
                                   -sum[2] * 9.5367431640625e-7f, -sum[3] * 9.5367431640625e-7f};   // 2^-20
            lds_bsc[blk] = __builtin_amdgcn_ldexpf(1.f, 20 - e);
        }
    }
}

}  // namespace

// The launch: a group of matrices (their 16-row tiles numbered across the group) in
// segments that each share one activation (MvSegs in mat_vec_common.h).  Each workgroup
// belongs to one segment and takes a contiguous range of its tiles.  The activation is
// staged in LDS one window of ws stages (16 ws blocks) at a time: phase p multiplies
// stages [p ws, (p + 1) ws) of every tile of the workgroup, and a tile's sum over the
// phases is kept in LDS (lds_tacc) between them, added in phase order.  Within a phase
// the (tile, stage) items are split evenly over the waves in tile-major order; a tile
// whose stages fall to two waves is finished after the phase's barrier by the wave that
// holds its last stage, adding the earlier waves' partials in wave order.  Every order of
// addition is fixed by the launch's geometry, so a call's results do not change from run
// to run.
struct BcIt {
    int tile, st;   // a (tile, stage) item
};

template <int NC, typename XT, bool EXACT>
__global__ __launch_bounds__(kMvStreamMaxWaves * 64)
__attribute__((amdgpu_waves_per_eu(4))) void mat_vec_bcast(MvGroup grp, MvSegs segs) {
    static_assert(NC == 1 || NC == 2, "one or two activation columns");
    static_assert(!EXACT || NC == 1, "exact mode: one column");
    constexpr int NR = EXACT ? 4 : 2 * NC;   // A rows: 4 limbs, or hi and lo per column
    const int WAVES = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));   // 4..16, chosen by the host

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int xcap = segs.xcap;
    uint8_t *lds_w = smem;                                                          // WAVES x kBcWaveLds
    float2_t *lds_part = reinterpret_cast<float2_t *>(smem + WAVES * kBcWaveLds);   // WAVES x 64
    half4_t *lds_x = reinterpret_cast<half4_t *>(lds_part + WAVES * 64);            // xcap x 16 x NR
    float4_t *lds_bs = reinterpret_cast<float4_t *>(lds_x + xcap * 16 * NR);        // exact mode: xcap
    float *lds_bsc = reinterpret_cast<float *>(lds_bs + (EXACT ? xcap : 0));        // exact mode: xcap
    float *lds_tacc = lds_bsc + (EXACT ? xcap : 0);                                 // tacc x 16 x NC
    __shared__ int lds_e[NC];
    __shared__ float lds_tmp[kMvStreamMaxWaves * NC];
    __shared__ int lds_part_tile[kMvStreamMaxWaves];   // lds_part: a wave's unfinished last tile
    static_assert(sizeof(lds_e) + sizeof(lds_tmp) + sizeof(lds_part_tile) <= kMvStreamStaticLds,
                  "static LDS reserve");

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, G = lane >> 4;   // this lane's row of the tile and quarter of the stage
    // ---- the kernel arguments this workgroup needs first, in one round trip: the tile
    // table, and per lane one segment record (lane & 7) and one matrix record (lane), read
    // as vectors; the workgroup's segment and its first tile's matrix are then picked with
    // ballots and lane reads.  (Read one after another as scalars -- the segments' first
    // workgroups, that segment's fields, then the matrix -- they were three dependent
    // round trips on the way to the first weight load of every launch.)
    const int t0v = load_tile_table(grp);   // the tile table, one entry per lane
    const uint8_t *const kargs = (const uint8_t *)__builtin_amdgcn_kernarg_segment_ptr();
    constexpr size_t kSegsOff = (sizeof(MvGroup) + alignof(MvSegs) - 1) / alignof(MvSegs) * alignof(MvSegs);
    const MvSeg *const segv = (const MvSeg *)(kargs + kSegsOff + offsetof(MvSegs, s)) + (lane & (kMvMaxSegs - 1));
    const MvProblem *const probv = (const MvProblem *)(kargs + offsetof(MvGroup, p)) + lane;
    const u32x4_t sv0 = *reinterpret_cast<const u32x4_t *>(segv);   // x, ldx
    const MvSeg sv = *segv;
    const u32x4_t pv0 = *reinterpret_cast<const u32x4_t *>(probv);  // w, y
    const u32x4_t pv1 = *reinterpret_cast<const u32x4_t *>(reinterpret_cast<const uint8_t *>(probv) + 16);   // ldy, M, tile0
    static_assert(offsetof(MvSeg, x) == 0 && offsetof(MvSeg, ldx) == 8, "segment record layout");
    static_assert(offsetof(MvProblem, w) == 0 && offsetof(MvProblem, y) == 8 && offsetof(MvProblem, ldy) == 16 &&
                  offsetof(MvProblem, M) == 24, "matrix record layout");
    static_assert(kMvMaxSegs == 8 && offsetof(MvSegs, s) == 0, "segment table");
    // segments hold ascending first workgroups (the first one 0): this workgroup's is the
    // last whose first workgroup it is not before
    const int sg = (int)__popcll(__ballot(lane < segs.n && lane < kMvMaxSegs && (int)blockIdx.x >= sv.wg0)) - 1;
    auto rl = [&](uint32_t v) { return (uint32_t)__builtin_amdgcn_readlane((int)v, sg); };
    // (pointers rebuilt from the lane reads pass through the global address space, so that
    // the loads through them stay global loads rather than flat ones)
    typedef const uint8_t __attribute__((address_space(1))) *gbytes;
    auto gptr = [](uint32_t lo, uint32_t hi) {
        return (const uint8_t *)(gbytes)(uintptr_t)(((uint64_t)hi << 32) | lo);
    };
    auto rli = [&](int v) { return __builtin_amdgcn_readlane(v, sg); };
    const XT *__restrict__ x = reinterpret_cast<const XT *>(gptr(rl(sv0.x), rl(sv0.y)));
    const int64_t ldx = (int64_t)(((uint64_t)rl(sv0.w) << 32) | rl(sv0.z));
    const MvSeg seg{x, ldx, rli(sv.nb), rli(sv.ws), rli(sv.tile0), rli(sv.tile1), rli(sv.wg0), rli(sv.wgs), rli(sv.q),
                    rli(sv.r), rl(sv.mag_w), rl(sv.mag_last)};
    const int nb = seg.nb, W = seg.ws;
    const int ns = (nb + kBcSB - 1) / kBcSB;
    const int P = (ns + W - 1) / W;
    const uint32_t rowbytes = (uint32_t)nb * kBlockBytes;
    const bool ragged = (nb % kBcSB) != 0;   // nb % 8 == 0: the last stage of a row then holds 8 blocks
    // (no divisions: the host splits the tiles, the waves are a power of two and the
    // stages of a window divide by a multiply-high; a division costs hundreds of cycles
    // on the path to the first load)
    const int bw = (int)blockIdx.x - seg.wg0;
    const int tb0 = seg.tile0 + bw * seg.q + min(bw, seg.r);
    const int nt = seg.q + (bw < seg.r ? 1 : 0);
    const int lw = __builtin_ctz((unsigned)WAVES);

    // Chunk q*64 + lane of a stage (chunks past the 288 repeat the last one): row
    // c / 18, bytes 16(c % 18) .. +15 of the row's 288.  Byte b of a row belongs to
    // quarter b / 72 and is parked at row * kBcRS + 80 (b / 72) + b % 72; a chunk's
    // two 8-byte halves are parked separately (at most one chunk per quarter boundary
    // splits, and 72 is a multiple of 8).  (The chunk's row and column are recomputed
    // where needed rather than kept in registers.)
    auto chunk_rc = [&](int q, int &crow, int &ccol) {
        const int c = min(q * 64 + lane, kBcNCH - 1);
        crow = c / kBcCPR;
        ccol = c - crow * kBcCPR;
    };
    uint32_t pk0[kBcCH], pk1[kBcCH];   // LDS byte offsets of the chunk's two halves
#pragma unroll
    for (int q = 0; q < kBcCH; ++q) {
        int crow, ccol;
        chunk_rc(q, crow, ccol);
        const int b0 = 16 * ccol, b1 = b0 + 8;
        pk0[q] = (uint32_t)(wave * kBcWaveLds + crow * kBcRS + b0 + 8 * (b0 / 72));
        pk1[q] = (uint32_t)(wave * kBcWaveLds + crow * kBcRS + b1 + 8 * (b1 / 72));
    }

    // Byte offsets of this lane's chunks from the first row of the tile being loaded;
    // rows past the matrix end are clamped to its last row (their outputs are never
    // stored).  Recomputed whenever the loads move to a new tile.
    uint32_t off[kBcCH];
    const uint8_t *ld_base = nullptr;   // first byte of the tile being loaded (uniform)
    int ld_tile = -1, ld_rows = -1;
    TileCursor ld_cur;
    {   // the first tile's matrix from the records read above
        ld_cur.idx = find_problem(t0v, tb0);
        auto rp = [&](uint32_t v) { return (uint32_t)__builtin_amdgcn_readlane((int)v, ld_cur.idx); };
        ld_cur.r = TileRef{gptr(rp(pv0.x), rp(pv0.y)),
                           reinterpret_cast<float *>(((uint64_t)rp(pv0.w) << 32) | rp(pv0.z)),
                           (int64_t)(((uint64_t)rp(pv1.y) << 32) | rp(pv1.x)), (int)rp(pv1.z), 0};
        ld_cur.t0 = __builtin_amdgcn_readlane(t0v, ld_cur.idx);
        ld_cur.t1 = ld_cur.idx + 1 < kMvMaxGroup ? __builtin_amdgcn_readlane(t0v, ld_cur.idx + 1) : 0x7fffffff;
    }
#define Q2_0_SET_LOAD_TILE(TILE)                                                                   \
    {                                                                                              \
        const TileRef tr_ = cursor_tile<kBcRows>(grp, t0v, ld_cur, (TILE));                        \
        ld_base = tr_.w + (int64_t)tr_.m0 * rowbytes;                                              \
        const int rows_ = min(tr_.M - tr_.m0, kBcRows);                                            \
        if (rows_ != ld_rows) {   /* only a matrix's last tile clamps */                           \
            _Pragma("unroll") for (int q = 0; q < kBcCH; ++q) {                                   \
                int crow_, ccol_;                                                                  \
                chunk_rc(q, crow_, ccol_);                                                         \
                off[q] = (uint32_t)min(crow_, rows_ - 1) * rowbytes + 16u * (uint32_t)ccol_;       \
            }                                                                                      \
            ld_rows = rows_;                                                                       \
        }                                                                                          \
        ld_tile = (TILE);                                                                          \
    }
    // Every call issues kBcCH loads.  In the half stage at the end of a ragged row, chunks
    // past its 144 bytes load its last chunk again.
#define Q2_0_ISSUE(IT, REG)                                                                    \
    {                                                                                          \
        if ((IT).tile != ld_tile) Q2_0_SET_LOAD_TILE((IT).tile)                               \
        const uint8_t *sbase = ld_base + (uint32_t)(IT).st * (uint32_t)(kBcSB * kBlockBytes);  \
        if (ragged && (IT).st == ns - 1) {                                                     \
            _Pragma("unroll") for (int q = 0; q < kBcCH; ++q) {                                \
                int crow_, ccol_;                                                              \
                chunk_rc(q, crow_, ccol_);                                                     \
                const uint32_t o = off[q] - 16u * (uint32_t)max(ccol_ - (kBcCPR / 2 - 1), 0);  \
                REG[q] = *reinterpret_cast<const u32x4_t *>(sbase + o);                        \
            }                                                                                  \
        } else {                                                                               \
            _Pragma("unroll") for (int q = 0; q < kBcCH; ++q)                                  \
                REG[q] = *reinterpret_cast<const u32x4_t *>(sbase + off[q]);                   \
        }                                                                                      \
    }
#define Q2_0_PARK(REG)                                                                          \
    {                                                                                           \
        _Pragma("unroll") for (int q = 0; q < kBcCH; ++q) {                                    \
            *reinterpret_cast<u32x2a8_t *>(lds_w + pk0[q]) = u32x2a8_t{REG[q].x, REG[q].y};     \
            *reinterpret_cast<u32x2a8_t *>(lds_w + pk1[q]) = u32x2a8_t{REG[q].z, REG[q].w};     \
        }                                                                                       \
    }

    // results leave as acc * 2^-e of their column (exact mode scales per block instead);
    // hi/lo mode scales each column once, over all of K, so every phase uses one exponent
    if (!EXACT) column_exponents<NC>(x, ldx, nb * kBlockWeights, lds_e, lds_tmp, tid, WAVES * 64);
    const int ye0 = EXACT ? 0 : -lds_e[0], ye1 = EXACT ? 0 : -lds_e[NC - 1];
    const uint8_t *lq = lds_w + wave * kBcWaveLds + r * kBcRS + G * kBcQuarter;   // this lane's quarter
    // A operand of code dword u of block blk: entry (blk*16 + 4u + a)*NR + row, a and
    // row from the lane's place in its 16-lane group
    const half4_t *xl = lds_x + (4 * G * 16 + ((lane >> 2) & 3)) * NR + ((NR == 2) ? (lane & 1) : (lane & 3));
    const PairMasks pm;
    float acc_e[2] = {0.f, 0.f}, acc_o[2] = {0.f, 0.f};

    // A finished tile of phase p: the row's four quarter sums are added (in a fixed order,
    // so every lane of the row holds the same value); quarter 0's lanes add the earlier
    // phases' sum and keep the total for the next phase, or, in the last phase, store it.
    auto finish_tile = [&](int p, int tile, float *y, int64_t ldy, int M, int m0, float r0, float r1) {
        r0 += __shfl_xor(r0, 16);
        r0 += __shfl_xor(r0, 32);
        if (NC > 1) {
            r1 += __shfl_xor(r1, 16);
            r1 += __shfl_xor(r1, 32);
        }
        if (G == 0) {
            float *ta = lds_tacc + ((tile - tb0) * kBcRows + r) * NC;
            if (p > 0) {
                r0 = ta[0] + r0;
                if (NC > 1) r1 = ta[1] + r1;
            }
            if (p + 1 < P) {
                ta[0] = r0;
                if (NC > 1) ta[1] = r1;
            } else if (m0 + r < M) {
                y[m0 + r] = __builtin_amdgcn_ldexpf(r0, ye0);
                if (NC > 1) y[ldy + m0 + r] = __builtin_amdgcn_ldexpf(r1, ye1);
            }
        }
    };

    // One stage in flight per wave.  A second register set (exact mode has the registers for
    // it) measured no faster on the 8B decode launch (419 against 415 us with one) and 7 %
    // slower on the per-layer schedule, whose small launches leave many waves a single
    // item that the second set then loads twice.  Q2_0_ISSUE_NEXT loads the wave's next
    // item of the phase (the loop calls it only while one is left).
    u32x4_t ra[kBcCH];
    for (int p = 0; p < P; ++p) {   // the same trip count in every wave: the barriers need it
        const int sw0 = p * W;                               // first stage of the window
        const int sp = min(W, ns - sw0);
        const uint32_t mag = p + 1 < P ? seg.mag_w : seg.mag_last;   // divides by sp (below 2^28)
        const int blk0 = sw0 * kBcSB;
        // this wave's items of the phase: (tile, stage) pairs i0 .. i1-1 of the workgroup's
        // nt * sp, tile-major
        const uint64_t n_wg = (uint64_t)(uint32_t)nt * (uint32_t)sp;
        const uint32_t i0 = (uint32_t)((n_wg * (uint32_t)wave) >> lw);
        const int n = (int)((uint32_t)((n_wg * (uint32_t)(wave + 1)) >> lw) - i0);
        const uint32_t i0t = sp == 1 ? i0 : __umulhi(i0, mag);   // (the magic of 1 would be 2^32)
        const BcIt first{tb0 + (int)i0t, sw0 + (int)(i0 - i0t * (uint32_t)sp)};
        const bool pend_start = n > 0 && first.st != sw0;   // its first tile began in an earlier wave
        auto next_item = [&](BcIt it) {
            if (++it.st == sw0 + sp) {
                it.st = sw0;
                ++it.tile;
            }
            return it;
        };
        BcIt ld = first, last = first;
        int n_left = n;   // items of the phase not issued yet
#define Q2_0_ISSUE_NEXT(REG)                                                                   \
    {                                                                                          \
        if (n_left > 0) {                                                                      \
            last = ld;                                                                         \
            ld = next_item(ld);                                                                \
            --n_left;                                                                          \
        }                                                                                      \
        Q2_0_ISSUE(last, REG)                                                                  \
    }
        // the first stages are issued before the window is staged, so that their latency
        // overlaps the staging
        // (exact mode: the window's first activation loads go out before them, so that the
        // staging waits for those alone)
        const XT *const xw = x + (int64_t)blk0 * kBlockWeights;
        const int nbw = min(sp * kBcSB, nb - blk0);
        LimbLoads xld;
        if (EXACT) limbs_load(xw, nbw, 0, tid, WAVES * 64, xld);
        if (n > 0) Q2_0_ISSUE_NEXT(ra)
        if (EXACT) {
            limbs_convert(nbw, 0, tid, WAVES * 64, xld, lds_x, lds_bs, lds_bsc);
            for (int q0 = kLimbU * WAVES * 64; q0 < nbw * 16; q0 += kLimbU * WAVES * 64) {
                limbs_load(xw, nbw, q0, tid, WAVES * 64, xld);
                limbs_convert(nbw, q0, tid, WAVES * 64, xld, lds_x, lds_bs, lds_bsc);
            }
        } else
            stage_x_bcast<NC>(x + (int64_t)blk0 * kBlockWeights, ldx, min(sp * kBcSB, nb - blk0), lds_e, lds_x, tid,
                              WAVES * 64);
        __syncthreads();

        float2_t pend = {0.f, 0.f};
        bool has_pend = false;   // this wave holds the last stage of a tile begun in an earlier wave
        BcIt cur = first;
        TileCursor out_cur;
        cursor_init(grp, t0v, out_cur, first.tile);
        int out_m0 = (first.tile - out_cur.t0) * kBcRows;   // rows of the tile being computed

    // Decode the parked stage `cur`, finish its tile after the window's last stage, and
    // move on within the phase; MORE: another item of the phase follows (on the last one
    // cur stays put).
#define Q2_0_COMPUTE(MORE)                                                                     \
    {                                                                                          \
        uint32_t R[4 * kBcCH];                                                                 \
        _Pragma("unroll") for (int i = 0; i < kBcCH; ++i) {                                   \
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(lq + 16 * i);                 \
            R[4 * i] = v.x; R[4 * i + 1] = v.y; R[4 * i + 2] = v.z; R[4 * i + 3] = v.w;        \
        }                                                                                      \
        /* this lane's blocks are cur.st*16 + 4G .. +3; the empty quarters of a ragged     */ \
        /* row's last stage read the window's blocks 0..3 instead (results discarded)      */ \
        const bool valid = cur.st * kBcSB + 4 * G < nb;                                        \
        const int sl = cur.st - sw0;                                                           \
        const int xoff = valid ? sl * kBcSB * 16 * NR : -4 * G * 16 * NR;                      \
        if (EXACT) {                                                                           \
            const int boff = valid ? sl * kBcSB + 4 * G : 0;                                   \
            bx_quarter(R, xl + xoff, lds_bs + boff, lds_bsc + boff, valid, acc_e, acc_o);      \
        } else {                                                                               \
            bc_quarter<NC>(R, xl + xoff, pm, valid, acc_e, acc_o);                             \
        }                                                                                      \
        if (cur.st == sw0 + sp - 1) {                                                          \
            const float r0 = acc_e[0] + acc_o[0], r1 = acc_e[1] + acc_o[1];                    \
            if (cur.tile == first.tile && pend_start) {                                        \
                pend = float2_t{r0, r1};                                                       \
                has_pend = true;                                                               \
            } else {                                                                           \
                finish_tile(p, cur.tile, out_cur.r.y, out_cur.r.ldy, out_cur.r.M, out_m0, r0, r1); \
            }                                                                                  \
            acc_e[0] = acc_e[1] = acc_o[0] = acc_o[1] = 0.f;                                   \
        }                                                                                      \
        if (MORE) {                                                                            \
            const BcIt nx_ = next_item(cur);                                                   \
            if (nx_.tile != cur.tile) {                                                        \
                cursor_tile<kBcRows>(grp, t0v, out_cur, nx_.tile);                             \
                out_m0 = (nx_.tile - out_cur.t0) * kBcRows;                                    \
            }                                                                                  \
            cur = nx_;                                                                         \
        }                                                                                      \
    }

        // Each step parks the stage that arrived, reissues the register set for the next
        // item and decodes the parked stage while those loads are in flight.  The last step
        // issues nothing: a wave cannot end before its loads return, and in small launches,
        // where many waves hold one or two items, a reload of the last one (to keep a fixed
        // number of loads in flight) landed on the launch's tail.  With one register set the
        // park waits for all of the wave's loads in any case.
        for (int k = 0; k < n; ++k) {
            Q2_0_PARK(ra)
            __builtin_amdgcn_wave_barrier();
            if (k + 1 < n) Q2_0_ISSUE_NEXT(ra)
            Q2_0_COMPUTE(k + 1 < n)
            __builtin_amdgcn_wave_barrier();
        }
#undef Q2_0_COMPUTE
#undef Q2_0_ISSUE_NEXT

        // An unfinished last tile (cur is the wave's last item) leaves its partial sums for
        // the wave that holds the tile's last stage of the window; that wave adds the earlier
        // waves' partials in order.
        const bool open_end = n > 0 && cur.st != sw0 + sp - 1;
        if (open_end) lds_part[wave * 64 + lane] = float2_t{acc_e[0] + acc_o[0], acc_e[1] + acc_o[1]};
        if (lane == 0) lds_part_tile[wave] = open_end ? cur.tile : -1;
        acc_e[0] = acc_e[1] = acc_o[0] = acc_o[1] = 0.f;
        __syncthreads();
        if (has_pend) {
            float r0 = 0.f, r1 = 0.f;
            for (int w = 0; w < wave; ++w) {
                if (lds_part_tile[w] == first.tile) {
                    const float2_t pp = lds_part[w * 64 + lane];
                    r0 += pp.x;
                    r1 += pp.y;
                }
            }
            const TileRef tr = tile_ref<kBcRows>(grp, t0v, first.tile);
            finish_tile(p, first.tile, tr.y, tr.ldy, tr.M, tr.m0, r0 + pend.x, r1 + pend.y);
        }
        __syncthreads();   // every wave is done with the window, lds_part and the accumulator
    }
#undef Q2_0_PARK
#undef Q2_0_ISSUE
#undef Q2_0_SET_LOAD_TILE
}

namespace {

// Window sizes: as many stages as the LDS left beside the wave tiles holds, up to 16 (the
// kernel's multiply-high division by the window's stages is exact for item counts below
// 2^28 up to 16 stages); where some row needs several windows, 16 KB stay free for the
// tile accumulator.  (16 waves: 8 stages, 6 when phased; 8 waves: 13 stages, e.g. a
// 12288-long row in one window; 4 waves: 16.)
constexpr int kBcMaxWindowStages = 16;
constexpr size_t kBcTaccReserve = 16 * 1024;

size_t x_bytes_per_block(int N, bool exact) { return exact ? 16 * 4 * 8 + 16 + 4 : (size_t)16 * 2 * N * 8; }

// Stages per window for a row of nb blocks: the fewest windows of at most cap stages, as
// even as possible.
int window_stages(int nb, int cap) {
    const int ns = (nb + kBcSB - 1) / kBcSB;
    const int P = (ns + cap - 1) / cap;
    return (ns + P - 1) / P;
}

}  // namespace

// Dynamic LDS of one workgroup of `waves` waves: the wave tiles, the waves' partial slots,
// the staged activation window (xcap blocks) and the tile accumulator (tacc tiles).  The
// kernel's static LDS (under kMvStreamStaticLds bytes) comes on top.
size_t mat_vec_bcast_lds(int N, int xcap, int tacc, int waves, bool exact) {
    return (size_t)waves * (kBcWaveLds + 64 * 8) + (size_t)xcap * x_bytes_per_block(N, exact) +
           (size_t)tacc * kBcRows * N * 4;
}

template <int NC, typename XT, bool EXACT>
static hipError_t launch_bcast_nc(const MvGroup &grp, const MvSegs &segs, hipStream_t s, int grid, int waves,
                                  size_t lds) {
    auto kern = mat_vec_bcast<NC, XT, EXACT>;
    // Raise the dynamic-LDS cap once per device.  Setting it is idempotent, so threads
    // that race past the flag set the same value; the flag itself is atomic.
    static std::atomic<bool> configured[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64 || !configured[dev].load(std::memory_order_acquire)) {
        hipFuncAttributes fa;
        e = hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(kern));
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)(160 * 1024 - fa.sharedSizeBytes));
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) configured[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * waves), lds, s, grp, segs);
    return hipGetLastError();
}

// grp counts tiles of kMvBcastRows rows; N is 1 or 2; every segment's rows and
// activation 16-byte aligned and nb % 8 == 0.  Workgroups go to the segments in
// proportion to their stages of work (a phased segment's stages weighted, below).
hipError_t launch_mat_vec_bcast(const MvGroup &grp, const MvSegDesc *d, int nsegs, Act xt, int N, hipStream_t s) {
    if (N < 1 || N > 2 || nsegs < 1 || nsegs > kMvMaxSegs) return hipErrorInvalidValue;
    const bool exact = N == 1;
    MvSegs segs;
    segs.n = nsegs;
    segs.xcap = 0;
    int64_t items = 0;
    int ns_max = 0;
    for (int i = 0; i < nsegs; ++i) {
        if (d[i].nb % 8 != 0 || d[i].tile1 <= d[i].tile0) return hipErrorInvalidValue;
        const int ns = (d[i].nb + kBcSB - 1) / kBcSB;
        ns_max = std::max(ns_max, ns);
        items += (int64_t)(d[i].tile1 - d[i].tile0) * ns;
    }
    // Waves per workgroup: 16 (one workgroup per CU) while an item for every wave still
    // leaves a workgroup per CU, else 8, and small launches then leave some waves without
    // an item.  Not 4: the workgroup's threads stage the whole activation window, and at 4
    // waves a 4096-long row takes each thread two rounds of loads and conversion (~2 us on
    // every launch's path, measured; 3 % of a per-layer decode).
    int waves = kMvStreamMaxWaves;   // a power of two (the kernel splits work by shifts)
    while (waves > 8 && (items + waves - 1) / waves < 256) waves /= 2;
    // windows: whole rows where the LDS left holds them all, else at most cap_phased stages
    const int64_t per_stage = (int64_t)kBcSB * (int64_t)x_bytes_per_block(N, exact);
    const int64_t avail = (int64_t)160 * 1024 - (int64_t)waves * (kBcWaveLds + 64 * 8) - (int64_t)kMvStreamStaticLds;
    const int cap_full = (int)std::min<int64_t>(kBcMaxWindowStages, avail / per_stage);
    const int cap_phased =
        (int)std::min<int64_t>(kBcMaxWindowStages, (avail - (int64_t)kBcTaccReserve) / per_stage);
    const int cap = ns_max <= cap_full ? cap_full : cap_phased;
    if (cap < 1) return hipErrorInvalidValue;
    bool phased = false;
    for (int i = 0; i < nsegs; ++i) {
        MvSeg &g = segs.s[i];
        g.x = d[i].x;
        g.ldx = d[i].ldx;
        g.nb = d[i].nb;
        g.ws = window_stages(d[i].nb, cap);
        g.tile0 = d[i].tile0;
        g.tile1 = d[i].tile1;
        const int ns = (g.nb + kBcSB - 1) / kBcSB;
        segs.xcap = std::max(segs.xcap, std::min(g.ws * kBcSB, g.nb));
        phased = phased || g.ws < ns;
    }
    for (int i = nsegs; i < kMvMaxSegs; ++i) segs.s[i] = MvSeg{nullptr, 0, 8, 1, 0, 0, 0x7fffffff, 0, 0, 0, 1u, 1u};
    const size_t fixed = mat_vec_bcast_lds(N, segs.xcap, 0, waves, exact) + kMvStreamStaticLds;
    if (fixed > 160 * 1024) return hipErrorInvalidValue;
    // the tile accumulator of phased segments takes what LDS is left
    const int tacc_cap = phased ? (int)((160 * 1024 - fixed) / ((size_t)kBcRows * N * 4)) : 0;
    if (phased && tacc_cap < 1) return hipErrorInvalidValue;
    const int per_cu = std::max(1, (int)((160 * 1024) / fixed));
    // at least a workgroup per CU where the tiles allow (some waves may then get no item)
    int64_t want = std::min<int64_t>(std::max<int64_t>((items + waves - 1) / waves, 256), 256 * (int64_t)per_cu);
    // Workgroups go to the segments in proportion to their stages, a stage of a phased
    // segment (several windows: its activation staged again, its tile sums kept in LDS)
    // counted as 1.036: measured per workgroup, with equal bytes each, the decode step's
    // K = 12288 workgroups (two windows) ended 3.6 % after its K = 4096 ones (one window),
    // and weighting them so took that launch from 419.5 to 414.8 us.
    constexpr int64_t kStageWeight = 1000, kPhasedStageWeight = 1036;
    auto seg_work = [&](const MvSeg &g) {
        const int64_t ns_ = (g.nb + kBcSB - 1) / kBcSB;
        return (int64_t)(g.tile1 - g.tile0) * ns_ * (g.ws < ns_ ? kPhasedStageWeight : kStageWeight);
    };
    int64_t work = 0;
    for (int i = 0; i < nsegs; ++i) work += seg_work(segs.s[i]);
    int wg = 0, tacc = 0;
    for (int i = 0; i < nsegs; ++i) {
        MvSeg &g = segs.s[i];
        const int T = g.tile1 - g.tile0;
        const int ns = (g.nb + kBcSB - 1) / kBcSB;
        int64_t n = (want * seg_work(g) + work / 2) / work;    // share of the workgroups
        n = std::max<int64_t>(1, std::min<int64_t>(n, T));     // at least one tile each
        if (g.ws < ns) n = std::max<int64_t>(n, (T + tacc_cap - 1) / tacc_cap);
        if ((int64_t)wg + n > 0x7fffffff) return hipErrorInvalidValue;
        g.wg0 = wg;
        g.wgs = (int)n;
        g.q = (int)(T / n);
        g.r = (int)(T % n);
        wg += (int)n;
        if (g.ws < ns) tacc = std::max(tacc, (int)((T + n - 1) / n));
        // the kernel divides item counts below 2^28 by at most 16 stages with a multiply-high
        if ((int64_t)(g.q + 1) * g.ws >= ((int64_t)1 << 28)) return hipErrorInvalidValue;
        const int last = ns - (ns + g.ws - 1) / g.ws * g.ws + g.ws;   // stages of the last window
        g.mag_w = (uint32_t)(0xffffffffu / (uint32_t)g.ws) + 1u;
        g.mag_last = (uint32_t)(0xffffffffu / (uint32_t)last) + 1u;
    }
    segs.tacc = tacc;
    const size_t lds = mat_vec_bcast_lds(N, segs.xcap, tacc, waves, exact);
    return with_act(xt, [&](auto tag) -> hipError_t {
        using XT = decltype(tag);
        if (N == 2) return launch_bcast_nc<2, XT, false>(grp, segs, s, wg, waves, lds);
        return launch_bcast_nc<1, XT, true>(grp, segs, s, wg, waves, lds);
    });
}

}  // namespace q2_0
