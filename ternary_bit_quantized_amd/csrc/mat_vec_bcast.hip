// Persistent mat-vec for N = 1, 2 on the gfx950 matrix cores' 16-block 4x4x4
// product, with the activation broadcast from registers inside groups of 16 lanes.
//
// Arithmetic as in the other MFMA mat-vec kernels (bisque.today "WebGPU: add Q2_0
// support", the matrix-vector paragraph: per 64-weight block the sum of (q - 1) * x,
// multiplied by the block scale once): exact fp16 (q - 1) from the pair decode, the
// activation as an fp16 hi/lo pair scaled per column by a power of two, products
// exact, sums in f32.
//
// The product: v_mfma_f32_4x4x4_16b_f16 runs 16 independent 4x4x4 products, block b
// on lanes 4b..4b+3; with CBSZ = 2 the blocks form 4 groups of 4 (16 lanes each), and
// every block of group G takes the A operand of block 4G + ABID.  Lane 16G + 4a + i
// holds A row i of chunk a, a chunk being 4 activations, the rows x hi, x lo (N = 1;
// rows 2, 3 repeat them) or column 0 hi, lo and column 1 hi, lo (N = 2).  One pair of
// VGPRs thus holds, for each group, the 16 activations of one code dword, and
// ABID = 0..3 on 4 successive products selects its chunks.  B column 16G + r is
// weight row r of the tile, i.e. the lane: group G's lanes decode the 16 rows' blocks
// of quarter G of the stage, and each lane accumulates its own (row, quarter) sum in
// D items 0..3.  The four quarters of a row are added once per tile by two lane
// exchanges.  Activation reads from LDS: one 8-byte read per code dword and lane, a
// quarter of what the 16x16x32 form needs; decode VALU: the pair decode only.
//
// Streaming as in mat_vec_stream.hip: work items (16-row tile, stage of 16 blocks),
// tile-major, split evenly over persistent workgroups and their waves; each wave keeps
// one stage in flight in registers (coalesced 16-byte loads, consecutive lanes on
// consecutive bytes of a row: 16 rows x 288 bytes, an access pattern that reads at
// the full rate of a contiguous stream) while it decodes the previous one from a
// wave-private LDS tile.  The park routes each 8-byte half of a loaded chunk to the
// LDS area of its quarter (80 bytes per quarter, 16-byte aligned), from which each lane
// reads its quarter with five 16-byte reads.  A tile whose stages are split between
// waves is finished after one barrier at the end, in stage order, so results are
// deterministic.
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
// xa: the activation operands of the 4 blocks x 4 code dwords; acc_e / acc_o accumulate
// even / odd blocks; a quarter outside the row (the empty half of a row's last stage
// when K/64 % 16 == 8) leaves them unchanged.
template <int NC>
__device__ __forceinline__ void bc_quarter(const uint32_t (&R)[20], const half4_t (&xa)[16], const PairMasks &pm,
                                           bool valid, float (&acc_e)[2], float (&acc_o)[2]) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int o = 9 * p;
        const uint32_t h0h7 = __builtin_amdgcn_perm(R[o + 4], R[o + 0], 0x05040302u);
        // scheduling fences keep the decode of one block next to its products (hoisted
        // ahead, the decoded halves of several blocks would not fit in registers)
        __builtin_amdgcn_sched_barrier(0);
        const float4_t se = bc_block(h0h7, R[o + 1], R[o + 2], R[o + 3], xa + 8 * p, pm);
        __builtin_amdgcn_sched_barrier(0);
        const float4_t so = bc_block(R[o + 5], R[o + 6], R[o + 7], R[o + 8], xa + 8 * p + 4, pm);
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
    const int items = nb * 16 * NC;
    for (int q = tid; q < items; q += nthreads) {
        const int n = q % NC, c = (q / NC) % 16, blk = q / (16 * NC);
        const int u = c >> 2, t = c & 3, odd = blk & 1;
        const XT *xb = x + n * ldx + (int64_t)blk * kBlockWeights + 2 * t;
        const float2_t a = load_act2(xb + 8 * half_lo(u, odd)), b = load_act2(xb + 8 * half_hi(u, odd));
        const int xe = lds_e[n];
        const float v[4] = {__builtin_amdgcn_ldexpf(a.x, xe), __builtin_amdgcn_ldexpf(b.x, xe),
                            __builtin_amdgcn_ldexpf(a.y, xe), __builtin_amdgcn_ldexpf(b.y, xe)};
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

// Exact-mode staging of one activation column for blocks 0..nb-1: limb entries
// (blk*16 + c)*4 + l (half4 of chunk c = 4u + t, limb l, in the weight order of
// bx_dword, each element times bx_factor), and per block bs = -2^-20 sum L per limb
// (NaN for limb 0 when the block holds a non-finite activation) and bsc = 2^(20-e).  One thread per chunk;
// the 16 chunks of a block sit in 16 consecutive lanes, which reduce the block's
// maximum and limb sums with lane exchanges.
template <typename XT>
__device__ __forceinline__ void stage_x_limbs(const XT *__restrict__ x, int nb, half4_t *lds_x, float4_t *lds_bs,
                                              float *lds_bsc, int tid, int nthreads) {
    const int items = nb * 16;
    for (int q0 = 0; q0 < items; q0 += nthreads) {   // the same trip count in every lane
        const int q = min(q0 + tid, items - 1);
        const bool act = q0 + tid < items;           // whole 16-lane groups are active or not
        const int c = q % 16, blk = q / 16;
        const int u = c >> 2, t = c & 3, odd = blk & 1;
        const XT *xb = x + (int64_t)blk * kBlockWeights + 2 * t;
        const float2_t a = load_act2(xb + 8 * half_lo(u, odd)), b = load_act2(xb + 8 * half_hi(u, odd));
        const float v[4] = {a.x, b.x, a.y, b.y};
        float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
        const bool finite = m <= 3.4028234663852886e38f;   // false for inf and NaN
        const int e = (finite && m > 0.f) ? 11 - __builtin_amdgcn_frexp_expf(m) : 0;
        float lim[4][4], sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float w = finite ? __builtin_amdgcn_ldexpf(v[k], e) : 0.f;
#pragma unroll
            for (int l = 0; l < 4; ++l) {
                const float L = __builtin_rintf(w);
                w = (w - L) * 2048.f;   // exact: the remainder of a rounded f32 and a power of two
                lim[l][k] = L;
                sum[l] += L;
            }
        }
        if (act) {
#pragma unroll
            for (int l = 0; l < 4; ++l) {
                half4_t h;
#pragma unroll
                for (int k = 0; k < 4; ++k) h[k] = (_Float16)(lim[l][k] * bx_factor(t, k));
                lds_x[(blk * 16 + c) * 4 + l] = h;
            }
        }
#pragma unroll
        for (int l = 0; l < 4; ++l)
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) sum[l] += __shfl_xor(sum[l], off);
        if (act && c == 0) {
            const float nan = __builtin_nanf("");
            lds_bs[blk] = float4_t{finite ? -sum[0] * 9.5367431640625e-7f : nan, -sum[1] * 9.5367431640625e-7f,
                                   -sum[2] * 9.5367431640625e-7f, -sum[3] * 9.5367431640625e-7f};   // 2^-20
            lds_bsc[blk] = __builtin_amdgcn_ldexpf(1.f, 20 - e);
        }
    }
}

}  // namespace

template <int NC, typename XT, bool EXACT>
__global__ __launch_bounds__(kMvStreamMaxWaves * 64)
__attribute__((amdgpu_waves_per_eu(4))) void mat_vec_bcast(MvGroup grp, int nb, const XT *__restrict__ x,
                                                     int64_t ldx) {
    static_assert(NC == 1 || NC == 2, "one or two activation columns");
    static_assert(!EXACT || NC == 1, "exact mode: one column");
    constexpr int NR = EXACT ? 4 : 2 * NC;   // A rows: 4 limbs, or hi and lo per column
    const int WAVES = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));   // 4..16, chosen by the host

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *lds_w = smem;                                                          // WAVES x kBcWaveLds
    float2_t *lds_part = reinterpret_cast<float2_t *>(smem + WAVES * kBcWaveLds);   // WAVES x 64
    half4_t *lds_x = reinterpret_cast<half4_t *>(lds_part + WAVES * 64);            // nb x 16 x NR
    float4_t *lds_bs = reinterpret_cast<float4_t *>(lds_x + nb * 16 * NR);          // exact mode: nb
    float *lds_bsc = reinterpret_cast<float *>(lds_bs + nb);                        // exact mode: nb
    __shared__ int lds_e[NC];
    __shared__ float lds_tmp[kMvStreamMaxWaves * NC];
    __shared__ int lds_part_tile[kMvStreamMaxWaves];   // lds_part: a wave's unfinished last tile
    static_assert(sizeof(lds_e) + sizeof(lds_tmp) + sizeof(lds_part_tile) <= kMvStreamStaticLds,
                  "static LDS reserve");

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, G = lane >> 4;   // this lane's row of the tile and quarter of the stage
    const int total = grp.total_tiles;
    const int t0v = load_tile_table(grp);   // the tile table, one entry per lane
    const int ns = (nb + kBcSB - 1) / kBcSB;
    const uint32_t rowbytes = (uint32_t)nb * kBlockBytes;
    const bool ragged = (nb % kBcSB) != 0;   // nb % 8 == 0: the last stage of a row then holds 8 blocks

    // This workgroup's tiles [tb0, tb1) and this wave's items [i0, i1) among them.
    // (products and quotients without 64-bit integer divisions, which would cost
    // hundreds of instructions before the first load)
    const int tb0 = (int)mul_div(total, blockIdx.x, gridDim.x);
    const int tb1 = (int)mul_div(total, blockIdx.x + 1, gridDim.x);
    const int64_t n_wg = (int64_t)(tb1 - tb0) * ns;
    const int64_t i0 = mul_div(n_wg, wave, WAVES), i1 = mul_div(n_wg, wave + 1, WAVES);
    const int n_items = (int)(i1 - i0);
    const int64_t i0_tile = div_floor(i0, ns);
    const BcItem first{tb0 + (int)i0_tile, (int)(i0 - i0_tile * ns)};

    // Chunk q*64 + lane of a stage (chunks past the 288 repeat the last one): row
    // c / 18, bytes 16(c % 18) .. +15 of the row's 288.  Byte b of a row belongs to
    // quarter b / 72 and is parked at row * kBcRS + 80 (b / 72) + b % 72; a chunk's
    // two 8-byte halves are parked separately (at most one chunk per quarter boundary
    // splits, and 72 is a multiple of 8).
    int cr[kBcCH], cc[kBcCH];
    uint32_t pk0[kBcCH], pk1[kBcCH];   // LDS byte offsets of the chunk's two halves
#pragma unroll
    for (int q = 0; q < kBcCH; ++q) {
        const int c = min(q * 64 + lane, kBcNCH - 1);
        cr[q] = c / kBcCPR;
        cc[q] = c % kBcCPR;
        const int b0 = 16 * cc[q], b1 = b0 + 8;
        pk0[q] = (uint32_t)(wave * kBcWaveLds + cr[q] * kBcRS + b0 + 8 * (b0 / 72));
        pk1[q] = (uint32_t)(wave * kBcWaveLds + cr[q] * kBcRS + b1 + 8 * (b1 / 72));
    }

    // Byte offsets of this lane's chunks from the first row of the tile being loaded;
    // rows past the matrix end are clamped to its last row (their outputs are never
    // stored).  Recomputed whenever the loads move to a new tile.
    uint32_t off[kBcCH];
    const uint8_t *ld_base = nullptr;   // first byte of the tile being loaded (uniform)
    int ld_tile = -1, ld_rows = -1;
    TileCursor ld_cur;
    cursor_init(grp, t0v, ld_cur, first.tile);
#define Q2_0_SET_LOAD_TILE(TILE)                                                                   \
    {                                                                                              \
        const TileRef tr_ = cursor_tile<kBcRows>(grp, t0v, ld_cur, (TILE));                             \
        ld_base = tr_.w + (int64_t)tr_.m0 * rowbytes;                                              \
        const int rows_ = min(tr_.M - tr_.m0, kBcRows);                                            \
        if (rows_ != ld_rows) {   /* only a matrix's last tile clamps */                           \
            _Pragma("unroll") for (int q = 0; q < kBcCH; ++q)                                     \
                off[q] = (uint32_t)min(cr[q], rows_ - 1) * rowbytes + 16u * (uint32_t)cc[q];       \
            ld_rows = rows_;                                                                       \
        }                                                                                          \
        ld_tile = (TILE);                                                                          \
    }
    // Every call issues exactly kBcCH loads (items past the wave's range reload the
    // current one), so the wait counts before each park stay exact.  In the half stage
    // at the end of a ragged row, chunks past its 144 bytes load its last chunk again.
#define Q2_0_ISSUE(IT, REG)                                                                    \
    {                                                                                          \
        if ((IT).tile != ld_tile) Q2_0_SET_LOAD_TILE((IT).tile)                               \
        const uint8_t *sbase = ld_base + (uint32_t)(IT).st * (uint32_t)(kBcSB * kBlockBytes);  \
        if (ragged && (IT).st == ns - 1) {                                                     \
            _Pragma("unroll") for (int q = 0; q < kBcCH; ++q) {                                \
                const uint32_t o = off[q] - 16u * (uint32_t)max(cc[q] - (kBcCPR / 2 - 1), 0);  \
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

    auto next_item = [&](BcItem it) {
        BcItem n{it.tile, it.st + 1};
        if (n.st == ns) { n.st = 0; n.tile += 1; }
        return n;
    };

    // Stages in flight per wave: two in exact mode (its registers allow a second set),
    // one otherwise.  Q2_0_ISSUE_NEXT loads the wave's next item, or once all are issued
    // the last one again, so that every call issues exactly kBcCH loads and the wait
    // counts before each park stay exact.  The first stages are issued before x is
    // staged, so their latency overlaps the staging.
    constexpr int DEPTH = EXACT ? 2 : 1;
    BcItem ld = first, last = first;
    int n_left = n_items;   // items not issued yet
#define Q2_0_ISSUE_NEXT(REG)                                                                   \
    {                                                                                          \
        if (n_left > 0) {                                                                      \
            last = ld;                                                                         \
            ld = next_item(ld);                                                                \
            --n_left;                                                                          \
        }                                                                                      \
        Q2_0_ISSUE(last, REG)                                                                  \
    }
    u32x4_t ra[kBcCH], rb[kBcCH];
    if (n_items > 0) {
        Q2_0_ISSUE_NEXT(ra)
        if (DEPTH == 2) Q2_0_ISSUE_NEXT(rb)
    }

    if (EXACT) {
        stage_x_limbs(x, nb, lds_x, lds_bs, lds_bsc, tid, WAVES * 64);
    } else {
        column_exponents<NC>(x, ldx, nb * kBlockWeights, lds_e, lds_tmp, tid, WAVES * 64);
        stage_x_bcast<NC>(x, ldx, nb, lds_e, lds_x, tid, WAVES * 64);
    }
    __syncthreads();

    // results leave as acc * 2^-e of their column (exact mode scales per block instead)
    const int ye0 = EXACT ? 0 : -lds_e[0], ye1 = EXACT ? 0 : -lds_e[NC - 1];
    const uint8_t *lq = lds_w + wave * kBcWaveLds + r * kBcRS + G * kBcQuarter;   // this lane's quarter
    // A operand of code dword u of block blk: entry (blk*16 + 4u + a)*NR + row, a and
    // row from the lane's place in its 16-lane group
    const half4_t *xl = lds_x + (4 * G * 16 + ((lane >> 2) & 3)) * NR + ((NR == 2) ? (lane & 1) : (lane & 3));
    const PairMasks pm;
    float acc_e[2] = {0.f, 0.f}, acc_o[2] = {0.f, 0.f};
    float2_t pend = {0.f, 0.f};   // the first tile, when it started in an earlier wave
    bool has_pend = false;

    // The row's four quarter sums are added (in a fixed order, so every lane of the row
    // holds the same value) and stored by the lanes of quarter 0.
    auto store_tile = [&](const TileRef &tr, float r0, float r1) {
        r0 += __shfl_xor(r0, 16);
        r0 += __shfl_xor(r0, 32);
        if (NC > 1) {
            r1 += __shfl_xor(r1, 16);
            r1 += __shfl_xor(r1, 32);
        }
        const int row = tr.m0 + r;
        if (G == 0 && row < tr.M) {
            tr.y[row] = __builtin_amdgcn_ldexpf(r0, ye0);
            if (NC > 1) tr.y[tr.ldy + row] = __builtin_amdgcn_ldexpf(r1, ye1);
        }
    };

    TileCursor out_cur;
    cursor_init(grp, t0v, out_cur, first.tile);
    TileRef tr_out = cursor_tile<kBcRows>(grp, t0v, out_cur, first.tile);   // the tile being computed

    BcItem cur = first;

    // Decode the parked stage `cur`, finish its tile after the row's last stage, and
    // move on; MORE: another item follows.
#define Q2_0_COMPUTE(MORE)                                                                     \
    {                                                                                          \
        uint32_t R[4 * kBcCH];                                                                 \
        _Pragma("unroll") for (int i = 0; i < kBcCH; ++i) {                                   \
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(lq + 16 * i);                 \
            R[4 * i] = v.x; R[4 * i + 1] = v.y; R[4 * i + 2] = v.z; R[4 * i + 3] = v.w;        \
        }                                                                                      \
        /* this lane's blocks are cur.st*16 + 4G .. +3; the empty quarters of a ragged     */ \
        /* row's last stage read blocks 0..3 instead (their results are discarded)         */ \
        const bool valid = cur.st * kBcSB + 4 * G < nb;                                        \
        const int xoff = valid ? cur.st * kBcSB * 16 * NR : -4 * G * 16 * NR;                  \
        if (EXACT) {                                                                           \
            const int boff = valid ? cur.st * kBcSB + 4 * G : 0;                               \
            bx_quarter(R, xl + xoff, lds_bs + boff, lds_bsc + boff, valid, acc_e, acc_o);      \
        } else {                                                                               \
            half4_t xa[16];                                                                    \
            _Pragma("unroll") for (int i = 0; i < 16; ++i) xa[i] = xl[xoff + 4 * i * NR];     \
            bc_quarter<NC>(R, xa, pm, valid, acc_e, acc_o);                                    \
        }                                                                                      \
        if (cur.st == ns - 1) {                                                                \
            const float r0 = acc_e[0] + acc_o[0], r1 = acc_e[1] + acc_o[1];                    \
            if (cur.tile == first.tile && first.st != 0) {                                     \
                pend = float2_t{r0, r1};                                                       \
                has_pend = true;                                                               \
            } else {                                                                           \
                store_tile(tr_out, r0, r1);                                                    \
            }                                                                                  \
            acc_e[0] = acc_e[1] = acc_o[0] = acc_o[1] = 0.f;                                   \
        }                                                                                      \
        const BcItem nx_ = next_item(cur);                                                     \
        if ((MORE) && nx_.tile != cur.tile) tr_out = cursor_tile<kBcRows>(grp, t0v, out_cur, nx_.tile); \
        cur = nx_;                                                                             \
    }

    // Each step parks the stage that arrived in one register set, reissues that set for
    // the item DEPTH ahead and decodes the parked stage while the other loads are in
    // flight.  No exit in the middle of a loop, which keeps the compiler's memory wait
    // counts exact.
    if (DEPTH == 1) {
        for (int k = 0; k < n_items; ++k) {
            Q2_0_PARK(ra)
            __builtin_amdgcn_wave_barrier();
            Q2_0_ISSUE_NEXT(ra)
            Q2_0_COMPUTE(k + 1 < n_items)
            __builtin_amdgcn_wave_barrier();
        }
    } else {
        for (int k = 0; k < n_items; k += 2) {
            Q2_0_PARK(ra)
            __builtin_amdgcn_wave_barrier();
            Q2_0_ISSUE_NEXT(ra)
            Q2_0_COMPUTE(k + 1 < n_items)
            __builtin_amdgcn_wave_barrier();
            Q2_0_PARK(rb)
            __builtin_amdgcn_wave_barrier();
            Q2_0_ISSUE_NEXT(rb)
            if (k + 1 < n_items) Q2_0_COMPUTE(k + 2 < n_items)
            __builtin_amdgcn_wave_barrier();
        }
    }
#undef Q2_0_COMPUTE
#undef Q2_0_ISSUE_NEXT
#undef Q2_0_PARK
#undef Q2_0_ISSUE
#undef Q2_0_SET_LOAD_TILE

    // An unfinished last tile leaves its partial sums for the wave that holds the
    // tile's last stage; that wave adds the earlier waves' partials in order.
    const int64_t last_tile = div_floor(i1 - 1, ns);
    const bool open_end = n_items > 0 && (i1 - 1 - last_tile * ns != ns - 1);
    if (open_end) lds_part[wave * 64 + lane] = float2_t{acc_e[0] + acc_o[0], acc_e[1] + acc_o[1]};
    if (lane == 0) lds_part_tile[wave] = open_end ? (tb0 + (int)last_tile) : -1;
    __syncthreads();
    if (has_pend) {
        float r0 = 0.f, r1 = 0.f;
        for (int w = 0; w < wave; ++w) {
            if (lds_part_tile[w] == first.tile) {
                const float2_t p = lds_part[w * 64 + lane];
                r0 += p.x;
                r1 += p.y;
            }
        }
        store_tile(tile_ref<kBcRows>(grp, t0v, first.tile), r0 + pend.x, r1 + pend.y);
    }
}

// Dynamic LDS of one workgroup of `waves` waves: the wave tiles, the waves' partial
// slots and the staged activation (16 chunks x 2N rows x 8 bytes per block).  The
// kernel's static LDS (under kMvStreamStaticLds bytes) comes on top.
size_t mat_vec_bcast_lds(int N, int nb, int waves, bool exact) {
    const size_t x_per_block = exact ? 16 * 4 * 8 + 16 + 4 : (size_t)16 * 2 * N * 8;
    return (size_t)waves * (kBcWaveLds + 64 * 8) + (size_t)nb * x_per_block;
}

// Workgroup size: the wave count (4..16) that keeps the most waves resident per CU
// given the LDS each workgroup needs and four waves per SIMD; ties go to fewer, larger
// groups.  0 if even 4 waves do not fit; *resident (optional) receives the waves per CU.
int mat_vec_bcast_waves(int N, int nb, bool exact, int *resident) {
    const int per_simd = 4;
    int best = 0, best_res = 0;
    for (int w = kMvStreamMaxWaves; w >= 4; --w) {
        const size_t lds = mat_vec_bcast_lds(N, nb, w, exact) + kMvStreamStaticLds;
        if (lds > 160 * 1024) continue;
        int wgs = (int)((160 * 1024) / lds);
        while (wgs > 0 && wgs * w > 4 * per_simd) --wgs;
        if (wgs * w > best_res) { best_res = wgs * w; best = w; }
    }
    if (resident) *resident = best_res;
    return best;
}

// Exact mode for N = 1 wherever its larger activation staging still leaves 12 or more
// resident waves per CU (K up to 8192); the hi/lo mode otherwise.
static bool use_exact(int N, int nb) {
    int resident = 0;
    return N == 1 && mat_vec_bcast_waves(1, nb, true, &resident) > 0 && resident >= 12;
}

int mat_vec_bcast_waves(int N, int nb, int *resident) {
    return mat_vec_bcast_waves(N, nb, use_exact(N, nb), resident);
}

template <int NC, typename XT, bool EXACT>
static hipError_t launch_bcast_nc(const MvGroup &grp, int nb, const XT *x, int64_t ldx, hipStream_t s, int grid,
                                  int waves) {
    const size_t lds = mat_vec_bcast_lds(NC, nb, waves, EXACT);
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
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * waves), lds, s, grp, nb, x, ldx);
    return hipGetLastError();
}

// grp counts tiles of kMvBcastRows rows; N is 1 or 2; rows and x 16-byte aligned, nb % 8 == 0.
hipError_t launch_mat_vec_bcast(const MvGroup &grp, int nb, const void *xv, Act xt, int64_t ldx, int N,
                                hipStream_t s) {
    if (N < 1 || N > 2 || nb % 8 != 0) return hipErrorInvalidValue;
    const bool exact = use_exact(N, nb);
    int waves = mat_vec_bcast_waves(N, nb, exact, nullptr);
    if (waves == 0) return hipErrorInvalidValue;
    // Small launches: fewer waves per workgroup until there is a workgroup per CU.
    const int64_t ns = (nb + kBcSB - 1) / kBcSB;
    const int64_t items = (int64_t)grp.total_tiles * ns;
    while (waves > 4 && (items + waves - 1) / waves < 256) waves = (waves + 1) / 2 < 4 ? 4 : (waves + 1) / 2;
    const size_t lds = mat_vec_bcast_lds(N, nb, waves, exact) + kMvStreamStaticLds;
    const int per_cu = (int)((160 * 1024) / lds);
    const int max_grid = 256 * (per_cu < 1 ? 1 : per_cu);
    // every wave gets at least about one stage; never more workgroups than tiles
    int64_t need = (items + waves - 1) / waves;
    if (need > grp.total_tiles) need = grp.total_tiles;
    const int grid = (int)(need < max_grid ? need : max_grid);
    return with_act(xt, [&](auto tag) -> hipError_t {
        using XT = decltype(tag);
        const XT *x = static_cast<const XT *>(xv);
        if (N == 2) return launch_bcast_nc<2, XT, false>(grp, nb, x, ldx, s, grid, waves);
        return exact ? launch_bcast_nc<1, XT, true>(grp, nb, x, ldx, s, grid, waves)
                     : launch_bcast_nc<1, XT, false>(grp, nb, x, ldx, s, grid, waves);
    });
}

}  // namespace q2_0
