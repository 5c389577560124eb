// Persistent streaming mat-vec for N = 1..8 on the gfx950 matrix cores.
//
// Same arithmetic as mat_vec_mfma.hip (block sums of (q - 1) * x formed on the
// matrix cores from exact fp16 (q - 1) and an fp16 hi/lo split of x, one multiply
// by the block scale per block; bisque.today "WebGPU: add Q2_0 support", the
// matrix-vector paragraph), organised for throughput on large or grouped launches:
//
//  * The activation columns for the whole of K are converted once per workgroup
//    into LDS, laid out as the MFMA A operand, behind a single barrier.
//  * After that each wave streams on its own, with no workgroup barrier: it walks
//    16-row tiles (tile = wave id, + total waves, ...), each over all of K in
//    stages of SB blocks.  Two stages are in flight in registers (coalesced
//    16-byte loads, consecutive lanes on consecutive bytes of a row) while a third
//    is decoded, so HBM latency hides behind the decode.  Weight bytes pass
//    through a wave-private LDS tile only to be regrouped per lane.
//  * Loads are branch-free: rows past the end of a matrix are clamped to its last
//    row (their outputs are never stored).
//  * One launch may cover several matrices that share K and the activation (for
//    example the q, k, v projections, or gate and up): tiles are numbered across
//    the group and a wave looks its matrix up once per tile.
//  * Every output is produced by one wave over the full K (no split), so results
//    are deterministic and independent of the group and grid.
#include "q2_0_internal.h"
#include "mat_vec_common.h"

namespace q2_0 {

namespace {

// The wave's current matrix and tile, all wave-uniform.
struct TileRef {
    const uint8_t *w;
    float *y;
    int64_t ldy;
    int M;
    int m0;
};

__device__ __forceinline__ TileRef tile_ref(const MvGroup &grp, int tile) {
    const MvProblem &p = grp.p[find_problem(grp, tile)];
    return TileRef{p.w, p.y, p.ldy, p.M, (tile - p.tile0) * kMvTile};
}

struct Item {
    int tile, st;
};

}  // namespace

template <int NC, int SB>
__global__ __launch_bounds__(512) void mat_vec_stream(MvGroup grp, int nb, const float *__restrict__ x,
                                                      int64_t ldx) {
    constexpr int NR = 2 * NC;
    constexpr int RSB = SB * kBlockBytes + 16;
    constexpr int CPR = SB * kBlockBytes / 16;
    constexpr int CH = (kMvTile * CPR + 63) / 64;
    constexpr int WAVES = 8;
    static_assert(RSB % 16 == 0 && SB % 8 == 0, "stage geometry");

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *lds_w = smem;                                                       // WAVES x 16 x RSB
    half8_t *lds_x = reinterpret_cast<half8_t *>(smem + WAVES * kMvTile * RSB);  // nb x 2 x 4 x NR

    const int tid = threadIdx.x;
    // the wave index is uniform: keep it (and all tile bookkeeping) in SGPRs
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, g = lane >> 4;
    const int total = grp.total_tiles;
    const int tw = gridDim.x * WAVES;
    const int first = blockIdx.x * WAVES + wave;
    const int ns = (nb + SB - 1) / SB;
    const int64_t rowbytes = (int64_t)nb * kBlockBytes;

    // Per-lane chunk geometry of a full stage: chunk q*64 + lane -> row r, 16-byte
    // column cc.  Chunks past the tile (r >= 16) load a duplicate and are not parked.
    int cr[CH], ccol[CH];
#pragma unroll
    for (int q = 0; q < CH; ++q) {
        const int c = q * 64 + lane;
        cr[q] = c / CPR;
        ccol[q] = c % CPR;
    }

    // work item i of this wave = (tile first + (i / ns) * tw, stage i % ns)
    auto next_item = [&](Item it) {
        Item n{it.tile, it.st + 1};
        if (n.st == ns) { n.st = 0; n.tile += tw; }
        return n;
    };
    auto issue = [&](Item it, const TileRef &tr, u32x4_t (&reg)[CH]) {
        const int sb = min(SB, nb - it.st * SB);
        const int cpr = sb * kBlockBytes / 16;
        const uint8_t *base = tr.w + (int64_t)it.st * SB * kBlockBytes;
#pragma unroll
        for (int q = 0; q < CH; ++q) {
            const int row = min(tr.m0 + min(cr[q], kMvTile - 1), tr.M - 1);
            const int cc = min(ccol[q], cpr - 1);
            reg[q] = *reinterpret_cast<const u32x4_t *>(base + (int64_t)row * rowbytes + 16 * cc);
        }
    };
    uint8_t *lw = lds_w + wave * kMvTile * RSB;
    auto park = [&](Item it, const u32x4_t (&reg)[CH]) {
        const int sb = min(SB, nb - it.st * SB);
        const int cpr = sb * kBlockBytes / 16;
#pragma unroll
        for (int q = 0; q < CH; ++q)
            if (cr[q] < kMvTile && ccol[q] < cpr)
                *reinterpret_cast<u32x4_t *>(lw + cr[q] * RSB + 16 * ccol[q]) = reg[q];
    };

    // Prefetch the first two stages before staging x, so their latency overlaps it.
    Item cur{first, 0};
    Item nxt = next_item(cur);
    TileRef tr_cur = tile_ref(grp, first < total ? first : 0);
    TileRef tr_nxt = (nxt.st == 0 && nxt.tile < total) ? tile_ref(grp, nxt.tile) : tr_cur;
    u32x4_t regA[CH], regB[CH];
    if (first < total) issue(cur, tr_cur, regA);
    if (nxt.tile < total) issue(nxt, tr_nxt, regB);

    stage_x_all<NC>(x, ldx, nb, lds_x, tid, WAVES * 64);
    __syncthreads();
    if (first >= total) return;

    const uint8_t *lw_row = lw + j * RSB;
    const int arow = g * NR + (j % NR);
    const uint32_t sel = (g == 0) ? 0x05040302u : 0x03020100u;
    const PairMasks pm;
    float acc0[2] = {0.f, 0.f}, acc1[2] = {0.f, 0.f};

    auto compute_and_store = [&](Item it, const TileRef &tr) {
        const int sb = min(SB, nb - it.st * SB);
        const half8_t *ax = lds_x + (it.st * SB * 2 * 4) * NR + arow;
        if (sb == SB) {
#pragma unroll
            for (int pp = 0; pp < SB / 2; ++pp)
                mv_block_pair<NC>(lw_row + 36 * pp, ax + (2 * pp) * 2 * 4 * NR, g, sel, pm, acc0, acc1);
        } else {
            for (int pp = 0; pp < sb / 2; ++pp)
                mv_block_pair<NC>(lw_row + 36 * pp, ax + (2 * pp) * 2 * 4 * NR, g, sel, pm, acc0, acc1);
        }
        if (it.st == ns - 1) {
            const int row = tr.m0 + j;
            if (row < tr.M) {
                if (2 * g < NC) tr.y[(int64_t)(2 * g) * tr.ldy + row] = acc0[0] + acc1[0];
                if (2 * g + 1 < NC) tr.y[(int64_t)(2 * g + 1) * tr.ldy + row] = acc0[1] + acc1[1];
            }
            acc0[0] = acc0[1] = acc1[0] = acc1[1] = 0.f;
        }
    };

    // Two register buffers alternate: park A, refill A two items ahead, compute; then B.
    // (Written out rather than as a lambda over a register-array reference, which the
    // compiler would otherwise keep in scratch.)
#define Q2_0_HALF_STEP(REG)                                                        \
    {                                                                              \
        park(cur, REG);                                                            \
        __builtin_amdgcn_wave_barrier();                                           \
        const Item ahead = next_item(nxt);                                         \
        TileRef tr_ahead = tr_nxt;                                                 \
        if (ahead.st == 0 && ahead.tile < total) tr_ahead = tile_ref(grp, ahead.tile); \
        if (ahead.tile < total) issue(ahead, tr_ahead, REG);                       \
        compute_and_store(cur, tr_cur);                                            \
        __builtin_amdgcn_wave_barrier();                                           \
        if (nxt.tile >= total) break;                                              \
        cur = nxt;                                                                 \
        tr_cur = tr_nxt;                                                           \
        nxt = ahead;                                                               \
        tr_nxt = tr_ahead;                                                         \
    }
    while (true) {
        Q2_0_HALF_STEP(regA)
        Q2_0_HALF_STEP(regB)
    }
#undef Q2_0_HALF_STEP
}

size_t mat_vec_stream_lds(int N, int nb) {
    return (size_t)8 * kMvTile * (kMvStreamSB * kBlockBytes + 16) + (size_t)nb * 2 * 4 * 2 * N * 16;
}

template <int NC>
static hipError_t launch_stream_nc(const MvGroup &grp, int nb, const float *x, int64_t ldx,
                                   hipStream_t s, int grid) {
    constexpr int SB = kMvStreamSB;
    const size_t lds = mat_vec_stream_lds(NC, nb);
    auto kern = mat_vec_stream<NC, SB>;
    // Raise the dynamic-LDS cap once per device (idempotent, so a race is harmless).
    static bool configured[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64 || !configured[dev]) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) configured[dev] = true;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(512), lds, s, grp, nb, x, ldx);
    return hipGetLastError();
}

hipError_t launch_mat_vec_stream(const MvGroup &grp, int nb, const float *x, int64_t ldx, int N,
                                 hipStream_t s) {
    const size_t lds = mat_vec_stream_lds(N, nb);
    const int per_cu = (int)((160 * 1024) / lds);
    const int max_grid = 256 * (per_cu < 1 ? 1 : per_cu);
    const int need = (grp.total_tiles + 7) / 8;
    const int grid = need < max_grid ? need : max_grid;
    switch (N) {
        case 1: return launch_stream_nc<1>(grp, nb, x, ldx, s, grid);
        case 2: return launch_stream_nc<2>(grp, nb, x, ldx, s, grid);
        case 3: return launch_stream_nc<3>(grp, nb, x, ldx, s, grid);
        case 4: return launch_stream_nc<4>(grp, nb, x, ldx, s, grid);
        case 5: return launch_stream_nc<5>(grp, nb, x, ldx, s, grid);
        case 6: return launch_stream_nc<6>(grp, nb, x, ldx, s, grid);
        case 7: return launch_stream_nc<7>(grp, nb, x, ldx, s, grid);
        case 8: return launch_stream_nc<8>(grp, nb, x, ldx, s, grid);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace q2_0
