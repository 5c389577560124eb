// K-split mat-vec for N = 1..8 on the gfx950 matrix cores, fp32-grade (used for
// single matrices too small to fill the chip with whole-K waves).
//
// What is computed follows the matrix-vector paragraph of bisque.today "WebGPU:
// add Q2_0 support": per block, the sum of (q - 1) * x over its 64 weights, then
// one multiply by the block scale d.  How it is computed is specific to gfx950:
//
//  * Weights.  A wave owns 16 rows.  Its rows' bytes are fetched with coalesced
//    16-byte loads (consecutive lanes read consecutive 16 B of a row) into
//    registers one stage ahead, then parked in a wave-private LDS tile.  Rows are
//    16-byte aligned (K/64 % 8 == 0), so a block pair is 9 aligned dwords:
//    D0 = [d_b | h0], D1..D3 = code halves h1..h6, D4 = [h7 | d_b+1], D5..D8 =
//    the four words of block b+1 (h_i = 8 codes of weights 8i..8i+7).  The
//    2-byte misalignment of even blocks is absorbed by pairing h0 with h7
//    (one v_perm_b32); every other code dword is read aligned.
//  * Decode.  A code dword holds two halves of 8 codes; codes at the same offset
//    s of both halves form an fp16 pair.  OR-ing the code into the mantissa under
//    the exponent 25-2s gives 2^(10-2s) + q exactly, and one packed subtract of
//    2^(10-2s) + 1 leaves q - 1 in {-1, 0, 1, 2} exactly: 2 VALU ops per 2 weights.
//  * Product.  v_mfma_f32_16x16x32_f16 with the activation as the A operand and
//    the weights as B: A row 2n is fp16(x_n) and row 2n+1 is fp16(x_n - fp16(x_n)),
//    so x = hi + lo to ~22 bits; products with (q - 1) are exact and accumulate in
//    f32.  The matrix core therefore performs the 64-term block sum and the
//    cross-lane reduction; per block the f32 result is scaled once by d.
//  * Activations are converted once per workgroup and stage into an LDS buffer
//    laid out exactly as the A operand.  A rows beyond 2N repeat valid rows and
//    their outputs are ignored.
//  * K split.  The four waves of a workgroup cover RG row tiles x KS slices of K;
//    slice partials are added in LDS in a fixed order (deterministic).
//
// Accuracy: each column is staged scaled by a power of two that takes its max |x|
// to [2^14, 2^15); the hi/lo split then errs <= 2^-22 |x| (at most 2^-39 of the
// column maximum for elements far below it), MFMA products are exact, and the f32
// chain is the MFMA sum plus K/128/KS block partials per accumulator (two
// accumulators alternate over blocks) -- inside the 1e-5 * sum|W x| bound.
#include "q2_0_internal.h"
#include "mat_vec_common.h"

namespace q2_0 {

constexpr int kTile = kMvTile;

// NC: activation columns; KS: K slices per workgroup (RG = 4 / KS row tiles);
// SB: blocks per stage.
// route.ids set (expert product, NC = 1): blockIdx.y is a (token, slot) pair p; its
// expert e = ids[p] selects the matrix at w + e * expert_bytes, its activation column is
// t (x_slots == 1) or p, and its result column p.  A pair with an id outside
// [0, n_expert) reads nothing: its workgroups write NaN into their rows of column p.
struct PairRoute {
    const int32_t *ids;
    int n_expert, n_used, x_slots;
    int64_t expert_bytes;
};

template <int NC, int KS, int SB, typename XT>
__global__ __launch_bounds__(256) void mat_vec_mfma(const uint8_t *__restrict__ w, int M, int nb,
                                                    const XT *__restrict__ x, int64_t ldx,
                                                    float *__restrict__ y, int64_t ldy, PairRoute route) {
    if (route.ids) {
        const int p = blockIdx.y;
        const int e = route.ids[p];
        if (e < 0 || e >= route.n_expert) {          // the whole workgroup
            constexpr int kRows = (4 / KS) * kTile;  // rows of this workgroup
            const int r1 = min(M, (int)blockIdx.x * kRows + kRows);
            for (int r = (int)blockIdx.x * kRows + (int)threadIdx.x; r < r1; r += 256)
                y[(int64_t)p * ldy + r] = __builtin_nanf("");
            return;
        }
        w += e * route.expert_bytes;
        x += (int64_t)(route.x_slots == 1 ? p / route.n_used : p) * ldx;
        y += (int64_t)p * ldy;
    }
    constexpr int RG = 4 / KS;
    constexpr int NR = 2 * NC;                      // A rows that carry data
    constexpr int RSB = SB * kBlockBytes + 16;       // LDS bytes per row per stage (16-B multiple)
    constexpr int CPR = SB * kBlockBytes / 16;       // 16-byte chunks per row per full stage
    constexpr int CH = (kTile * CPR + 63) / 64;      // chunks per lane per stage
    constexpr int XITEMS = KS * SB * 2 * 4 * NC;     // (slice, block, mfma, group, column) items
    constexpr int XI = (XITEMS + 255) / 256;         // items per thread
    static_assert(RSB % 16 == 0 && SB % 8 == 0, "stage geometry");

    __shared__ __attribute__((aligned(16))) uint8_t lds_w[4][kTile * RSB];
    __shared__ __attribute__((aligned(16))) half8_t lds_x[KS * SB * 2 * 4 * NR];
    __shared__ float lds_red[(KS > 1) ? 4 * kTile * NC : 1];
    __shared__ int lds_e[NC];
    __shared__ float lds_tmp[4 * NC];

    const int tid = threadIdx.x;
    // the wave index is uniform: keep it (and all tile bookkeeping) in SGPRs
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = wave / KS, ks = wave % KS;
    const int j = lane & 15, g = lane >> 4;
    const int m0 = (blockIdx.x * RG + rg) * kTile;
    const int nbw = nb / KS;                          // blocks in this wave's slice (multiple of 8)
    const int64_t rowbytes = (int64_t)nb * kBlockBytes;
    const int kb0 = ks * nbw;                          // first block of the slice
    const int nstage = (nbw + SB - 1) / SB;

    uint4 wreg[CH];
    XItem xreg[XI];

    // Stage st covers blocks [st*SB, st*SB + sb) of every slice; sb < SB only in the
    // last stage.  Chunk and item indices are laid out over a full stage (constant
    // divisors) and the ones beyond sb are skipped.
    auto issue_loads = [&](int st) {
        const int sb = min(SB, nbw - st * SB);
        const int cpr = sb * kBlockBytes / 16;
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            const int c = t * 64 + lane;
            const int r = c / CPR, cc = c % CPR;
            const int row = m0 + r;
            uint4 v = {0u, 0u, 0u, 0u};
            if (r < kTile && cc < cpr && row < M)
                v = *reinterpret_cast<const uint4 *>(w + (int64_t)row * rowbytes +
                                                     (int64_t)(kb0 + st * SB) * kBlockBytes + 16 * cc);
            wreg[t] = v;
        }
#pragma unroll
        for (int t = 0; t < XI; ++t) {
            const int q = t * 256 + tid;
            const int b = (q / (8 * NC)) % SB;
            if (q < XITEMS && b < sb) {
                const int n = q % NC, gg = (q / NC) % 4, mu = (q / (4 * NC)) % 2, sl = q / (8 * NC * SB);
                xreg[t] = load_x_item(x, ldx, sl * nbw + st * SB + b, mu, gg, n);
            }
        }
    };

    auto park = [&](int st) {
        const int sb = min(SB, nbw - st * SB);
        const int cpr = sb * kBlockBytes / 16;
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            const int c = t * 64 + lane;
            const int r = c / CPR, cc = c % CPR;
            if (r < kTile && cc < cpr)
                *reinterpret_cast<uint4 *>(&lds_w[wave][r * RSB + 16 * cc]) = wreg[t];
        }
#pragma unroll
        for (int t = 0; t < XI; ++t) {
            const int q = t * 256 + tid;
            const int b = (q / (8 * NC)) % SB;
            if (q < XITEMS && b < sb) {
                store_x_item(xreg[t], lds_e[q % NC], lds_x + (q / NC) * NR + 2 * (q % NC));
            }
        }
    };

    const PairMasks pm;
    float acc0[2] = {0.f, 0.f}, acc1[2] = {0.f, 0.f};   // even / odd blocks; columns 2g, 2g+1
    const int arow = g * NR + (j % NR);                   // A row this lane supplies (repeats past NR)
    const uint8_t *lw_row = &lds_w[wave][j * RSB];
    // Even block code dword: group 0 pairs h0 (high half of D0) with h7 (low half of D4);
    // the other groups read D_g as is.  v_perm_b32 selects bytes of {D4, D_g}.
    const uint32_t sel = (g == 0) ? 0x05040302u : 0x03020100u;

    issue_loads(0);
    column_exponents<NC>(x, ldx, nb * kBlockWeights, lds_e, lds_tmp, tid, 256);
    for (int st = 0; st < nstage; ++st) {
        park(st);
        __syncthreads();
        if (st + 1 < nstage) issue_loads(st + 1);
        const int sb = min(SB, nbw - st * SB);
        const half8_t *ax = &lds_x[(ks * SB * 2 * 4) * NR + arow];
#pragma unroll 2
        for (int p = 0; p < sb / 2; ++p)
            mv_block_pair<NC>(lw_row + 36 * p, ax + (2 * p) * 2 * 4 * NR, g, sel, pm, acc0, acc1);
        __syncthreads();
    }

    // Lane (j, g) holds rows m0 + j for columns 2g (index 0) and 2g + 1 (index 1).
    // (results leave as acc * 2^-e of their column)
    const float r0 = acc0[0] + acc1[0];
    const float r1 = acc0[1] + acc1[1];
    const int row = m0 + j;
    if (KS == 1) {
        if (row < M) {
            if (2 * g < NC) y[(int64_t)(2 * g) * ldy + row] = __builtin_amdgcn_ldexpf(r0, -lds_e[2 * g]);
            if (2 * g + 1 < NC)
                y[(int64_t)(2 * g + 1) * ldy + row] = __builtin_amdgcn_ldexpf(r1, -lds_e[2 * g + 1]);
        }
    } else {
        // slice partials -> LDS, then a fixed-order sum over the KS slices
        if (2 * g < NC) lds_red[((ks * RG + rg) * kTile + j) * NC + 2 * g] = r0;
        if (2 * g + 1 < NC) lds_red[((ks * RG + rg) * kTile + j) * NC + 2 * g + 1] = r1;
        __syncthreads();
        for (int o = tid; o < RG * kTile * NC; o += 256) {
            const int n = o % NC, rr = (o / NC) % kTile, tg = o / (NC * kTile);
            float sum = 0.f;
#pragma unroll
            for (int k = 0; k < KS; ++k) sum += lds_red[((k * RG + tg) * kTile + rr) * NC + n];
            const int orow = (blockIdx.x * RG + tg) * kTile + rr;
            if (orow < M) y[(int64_t)n * ldy + orow] = __builtin_amdgcn_ldexpf(sum, -lds_e[n]);
        }
    }
}

// Host-side choice of K slices: split K (up to 4 ways) while the grid has fewer than a
// workgroup per CU, or, for expert pairs, until a pair's workgroups reach 128 / pairs.
// Short calls pay for every wave they start: 8 pairs of 768 x 2048 took 5.7 us in 2
// slices (192 workgroups), 6.3 us in 4 and 6.6 us in 1; a 12288 x 4096 matrix ~1.9 us
// less in 2 slices (384 workgroups) than in 4.
template <int NC, typename XT>
static hipError_t launch_nc(const uint8_t *w, int M, int nb, const XT *x, int64_t ldx, float *y,
                            int64_t ldy, hipStream_t s, const PairRoute &route = PairRoute{}, int pairs = 1) {
    const int tiles = (M + kTile - 1) / kTile;
    int ks = 1;
    const int want = pairs > 1 ? (128 / pairs > 0 ? 128 / pairs : 1) : 256;
    const int maxks = (NC <= 4) ? 4 : 2;
    while (ks < maxks && (tiles + (4 / ks) - 1) / (4 / ks) < want && nb % (8 * ks * 2) == 0) ks *= 2;
    const int rg = 4 / ks;
    dim3 grid((unsigned)((tiles + rg - 1) / rg), (unsigned)pairs);
    constexpr int SB1 = (NC <= 4) ? 32 : 16;
    constexpr int SB2 = (NC <= 2) ? 32 : 16;
    constexpr int SB4 = (NC <= 1) ? 32 : ((NC <= 2) ? 16 : 8);
    if (ks == 1)
        mat_vec_mfma<NC, 1, SB1, XT><<<grid, 256, 0, s>>>(w, M, nb, x, ldx, y, ldy, route);
    else if (ks == 2)
        mat_vec_mfma<NC, 2, SB2, XT><<<grid, 256, 0, s>>>(w, M, nb, x, ldx, y, ldy, route);
    else if constexpr (NC <= 4)
        mat_vec_mfma<NC, 4, SB4, XT><<<grid, 256, 0, s>>>(w, M, nb, x, ldx, y, ldy, route);
    return hipGetLastError();
}

// Rows 16-byte aligned (K/64 % 8 == 0 and w aligned) and x aligned to four elements
// with ldx % 4 == 0, so that weight chunks and activation quads load as vectors.
bool mat_vec_mfma_eligible(const uint8_t *w, int64_t M, int nb, const void *x, Act xt, int64_t ldx) {
    return ((uintptr_t)w % 16 == 0) && (nb % 8 == 0) && ((uintptr_t)x % (4 * act_bytes(xt)) == 0) &&
           (ldx % 4 == 0) && M <= 0x7fffffff - 64;
}

hipError_t launch_mat_vec_mfma(const uint8_t *w, int64_t M, int nb, const void *xv, Act xt, int64_t ldx,
                               int N, float *y, int64_t ldy, hipStream_t s) {
    const int m = (int)M;
    return with_act(xt, [&](auto tag) -> hipError_t {
        using XT = decltype(tag);
        const XT *x = static_cast<const XT *>(xv);
        switch (N) {
            case 1: return launch_nc<1>(w, m, nb, x, ldx, y, ldy, s);
            case 2: return launch_nc<2>(w, m, nb, x, ldx, y, ldy, s);
            case 3: return launch_nc<3>(w, m, nb, x, ldx, y, ldy, s);
            case 4: return launch_nc<4>(w, m, nb, x, ldx, y, ldy, s);
            case 5: return launch_nc<5>(w, m, nb, x, ldx, y, ldy, s);
            case 6: return launch_nc<6>(w, m, nb, x, ldx, y, ldy, s);
            case 7: return launch_nc<7>(w, m, nb, x, ldx, y, ldy, s);
            case 8: return launch_nc<8>(w, m, nb, x, ldx, y, ldy, s);
            default: return hipErrorInvalidValue;
        }
    });
}

// Expert product with few tokens: one mat-vec (N = 1) per (token, slot) pair, the
// expert looked up on the GPU (fp32-grade, as q2_0_mul_mat gives for N <= 8).
hipError_t launch_mat_vec_mfma_pairs(const uint8_t *w, int64_t M, int nb, const void *xv, Act xt, int64_t ldx,
                                     const int32_t *ids, int n_expert, int n_used, int x_slots, int n_pairs,
                                     float *y, int64_t ldy, hipStream_t s) {
    const PairRoute route{ids, n_expert, n_used, x_slots, M * (int64_t)nb * kBlockBytes};
    return with_act(xt, [&](auto tag) -> hipError_t {
        using XT = decltype(tag);
        return launch_nc<1>(w, (int)M, nb, static_cast<const XT *>(xv), ldx, y, ldy, s, route, n_pairs);
    });
}

}  // namespace q2_0
