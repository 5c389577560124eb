// Persistent streaming mat-vec for N = 1..8 on the gfx950 matrix cores.
//
// Same arithmetic as mat_vec_mfma.hip (block sums of (q - 1) * x formed on the
// matrix cores from exact fp16 (q - 1) and an fp16 hi/lo split of x, one multiply
// by the block scale per block; bisque.today "WebGPU: add Q2_0 support", the
// matrix-vector paragraph), organised for throughput on large or grouped launches:
//
//  * The activation columns for the whole of K are converted once per workgroup
//    into LDS, laid out as the MFMA A operand, behind a single barrier; each
//    column is first scaled by a power of two that puts its max |x| just below
//    2^15, so the fp16 hi/lo split neither overflows nor loses bits to fp16's
//    subnormal range (the scale is undone on the results).  Where all of K does
//    not fit, the host runs the kernel over chunks of whole stages, one launch
//    each: a launch reads its chunk of every row (rows rowstride bytes apart) and
//    every chunk after the first adds its results to y, in chunk order.
//  * Work is a list of items (16-row tile, stage of SB blocks), tile-major.  Each
//    workgroup owns a contiguous run of tiles and each of its W waves (4 to 16,
//    chosen per shape so that the most waves stay resident within the LDS the
//    activation takes) a contiguous 1/W of that run's items, so every wave streams
//    the same number of stages to within one: no tail where a few waves finish a
//    last round alone.
//  * A wave streams on its own, with no barrier: one stage is in flight in
//    registers (coalesced 16-byte loads, consecutive lanes on consecutive bytes of
//    a row) while the previous one is decoded.  Weight bytes pass through a wave-private LDS
//    tile only to be regrouped per lane.  Loads are branch-free: rows past the end
//    of a matrix are clamped to its last row (their outputs are never stored).
//  * A tile whose stages are split between waves is finished after one barrier at
//    the end: the waves that hold its earlier stages leave their partial sums in
//    LDS, and the wave that holds its last stage adds them in stage order.  The
//    split depends only on the sizes and the grid, so results are deterministic.
//  * One launch may cover several matrices that share K and the activation (for
//    example the q, k, v projections, or gate and up): tiles are numbered across
//    the group and a wave looks its matrix up once per tile.
//  * A K too long for its activation to fit in LDS is run as consecutive launches over
//    chunks of whole stages: a launch reads nb blocks of each row (rows rowstride
//    bytes apart), and every chunk after the first adds its results to y, in chunk
//    order (deterministic; each chunk scales its activation by its own exponent).
#include <atomic>

#include "q2_0_internal.h"
#include "mat_vec_common.h"

namespace q2_0 {

namespace {

struct Item {
    int tile, st;
};

}  // namespace

template <int NC, int SB, typename XT>
__global__ __launch_bounds__(kMvStreamMaxWaves * 64)
__attribute__((amdgpu_waves_per_eu(4))) void mat_vec_stream(MvGroup grp, int nb, const XT *__restrict__ x,
                                                      int64_t ldx, uint32_t rowstride, int accumulate) {
    constexpr int NR = 2 * NC;
    constexpr int RSB = SB * kBlockBytes + 16;
    constexpr int CPR = SB * kBlockBytes / 16;        // 16-byte chunks per row of a full stage
    constexpr int NCHUNK = kMvTile * CPR;             // chunks of a full stage
    constexpr int CH = (NCHUNK + 63) / 64;            // chunks per lane
    constexpr int LAST_LANES = NCHUNK - 64 * (CH - 1);  // lanes whose last chunk is real
    const int WAVES = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));   // 4..16, chosen by the host
    static_assert(RSB % 16 == 0 && SB % 16 == 0, "stage geometry");

    constexpr int DUMMY = (64 - LAST_LANES) * 16;     // park slots for the lanes past the tile
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *lds_w = smem;   // WAVES x (16 x RSB + DUMMY)
    float2_t *lds_part = reinterpret_cast<float2_t *>(smem + WAVES * (kMvTile * RSB + DUMMY));  // WAVES x 64
    half8_t *lds_x = reinterpret_cast<half8_t *>(lds_part + WAVES * 64);                     // nb x 2 x 4 x NR
    __shared__ int lds_e[NC];
    __shared__ float lds_tmp[kMvStreamMaxWaves * NC];
    __shared__ int lds_part_tile[kMvStreamMaxWaves];   // lds_part: a wave's unfinished last tile
    static_assert(sizeof(lds_e) + sizeof(lds_tmp) + sizeof(lds_part_tile) <= kMvStreamStaticLds,
                  "static LDS reserve");

    const int tid = threadIdx.x;
    // the wave index is uniform: keep it (and all tile bookkeeping) in SGPRs
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, g = lane >> 4;
    const int total = grp.total_tiles;
    const int t0v = load_tile_table(grp);   // the tile table, one entry per lane
    const int ns = (nb + SB - 1) / SB;
    const uint32_t rowbytes = rowstride;   // bytes from one row to the next (nb blocks of each are read)
    const bool ragged = (nb % SB) != 0;   // the last stage of a row holds SB/2 blocks

    // This workgroup's tiles [tb0, tb1) and this wave's items [i0, i1) among them.
    // (products and quotients without 64-bit integer divisions, which would cost
    // hundreds of instructions before the first load)
    const int tb0 = (int)mul_div(total, blockIdx.x, gridDim.x);
    const int tb1 = (int)mul_div(total, blockIdx.x + 1, gridDim.x);
    const int64_t n_wg = (int64_t)(tb1 - tb0) * ns;
    const int64_t i0 = mul_div(n_wg, wave, WAVES), i1 = mul_div(n_wg, wave + 1, WAVES);
    const int n_items = (int)(i1 - i0);
    const int64_t i0_tile = div_floor(i0, ns);
    const Item first{tb0 + (int)i0_tile, (int)(i0 - i0_tile * ns)};

    // Per-lane chunk geometry of a stage: chunk q*64 + lane -> tile row cr, 16-byte column
    // cc, parked at lds_off.  In a half stage (SB/2 blocks) the chunks past its end load a
    // clamped duplicate, parked into the unused tail of the row.
    int cr[CH], cc[CH];
    uint32_t lds_off[CH];
#pragma unroll
    for (int q = 0; q < CH; ++q) {
        const int c = q * 64 + lane;
        cr[q] = min(c / CPR, kMvTile - 1);
        cc[q] = c % CPR;
        // chunks past the tile (lanes >= LAST_LANES of the last one) park in the wave's
        // dummy slots, so that every park is an unconditional store
        lds_off[q] = (uint32_t)(wave * (kMvTile * RSB + DUMMY) +
                                (c < NCHUNK ? (c / CPR) * RSB + 16 * cc[q] : kMvTile * RSB + 16 * (c - NCHUNK)));
    }

    // Byte offsets of this lane's chunks from the first row of the tile being loaded;
    // rows past the matrix end are clamped to its last row (their outputs are never
    // stored).  Recomputed whenever the loads move to a new tile.
    // (Macros rather than lambdas: a lambda writing a captured register array makes
    // the compiler keep the array in scratch.)
    uint32_t off[CH];
    const uint8_t *ld_base = nullptr;   // first byte of the tile being loaded (uniform)
    int ld_tile = -1, ld_rows = -1;
    TileCursor ld_cur;
    cursor_init(grp, t0v, ld_cur, first.tile);
#define Q2_0_SET_LOAD_TILE(TILE)                                                                   \
    {                                                                                              \
        const TileRef tr_ = cursor_tile<kMvTile>(grp, t0v, ld_cur, (TILE));                             \
        ld_base = tr_.w + (int64_t)tr_.m0 * rowbytes;                                              \
        const int rows_ = min(tr_.M - tr_.m0, kMvTile);                                            \
        if (rows_ != ld_rows) {   /* only a matrix's last tile clamps */                           \
            _Pragma("unroll") for (int q = 0; q < CH; ++q)                                        \
                off[q] = (uint32_t)min(cr[q], rows_ - 1) * rowbytes + 16u * (uint32_t)cc[q];       \
            ld_rows = rows_;                                                                       \
        }                                                                                          \
        ld_tile = (TILE);                                                                          \
    }

    auto next_item = [&](Item it) {
        Item n{it.tile, it.st + 1};
        if (n.st == ns) { n.st = 0; n.tile += 1; }
        return n;
    };
    // Every call issues CH loads; only the wave's own items are loaded (the last step issues
    // nothing, and with one register set each park waits for all of the wave's loads).
#define Q2_0_ISSUE(IT, REG)                                                                    \
    {                                                                                          \
        if ((IT).tile != ld_tile) Q2_0_SET_LOAD_TILE((IT).tile)                               \
        const uint8_t *sbase = ld_base + (uint32_t)(IT).st * (uint32_t)(SB * kBlockBytes);     \
        if (ragged && (IT).st == ns - 1) {                                                     \
            _Pragma("unroll") for (int q = 0; q < CH; ++q) {                                   \
                const uint32_t o = off[q] - 16u * (uint32_t)max(cc[q] - (CPR / 2 - 1), 0);     \
                REG[q] = *reinterpret_cast<const u32x4_t *>(sbase + o);                        \
            }                                                                                  \
        } else {                                                                               \
            _Pragma("unroll") for (int q = 0; q < CH; ++q)                                     \
                REG[q] = *reinterpret_cast<const u32x4_t *>(sbase + off[q]);                   \
        }                                                                                      \
    }
#define Q2_0_PARK(REG)                                                                          \
    {                                                                                           \
        _Pragma("unroll") for (int q = 0; q < CH; ++q)                                         \
            *reinterpret_cast<u32x4_t *>(lds_w + lds_off[q]) = REG[q];                          \
    }

    // The first stage is issued before x is staged, so its latency overlaps the staging;
    // on entering the loop exactly this stage is in flight, as on every later iteration.
    u32x4_t reg[CH];
    if (n_items > 0) Q2_0_ISSUE(first, reg)

    column_exponents<NC>(x, ldx, nb * kBlockWeights, lds_e, lds_tmp, tid, WAVES * 64);
    stage_x_all<NC>(x, ldx, nb, lds_e, lds_x, tid, WAVES * 64);
    __syncthreads();

    // results leave as acc * 2^-e of their column
    const int ye0 = -lds_e[min(2 * g, NC - 1)], ye1 = -lds_e[min(2 * g + 1, NC - 1)];
    const uint8_t *lw_row = lds_w + wave * (kMvTile * RSB + DUMMY) + j * RSB;
    const int arow = g * NR + (j % NR);
    const uint32_t sel = (g == 0) ? 0x05040302u : 0x03020100u;
    const PairMasks pm;
    float acc0[2] = {0.f, 0.f}, acc1[2] = {0.f, 0.f};
    float2_t pend = {0.f, 0.f};   // the first tile, when it started in an earlier wave
    bool has_pend = false;

    auto store_tile = [&](const TileRef &tr, float r0, float r1) {
        const int row = tr.m0 + j;
        if (row < tr.M) {
            float *const y0 = tr.y + (int64_t)(2 * g) * tr.ldy + row;
            float *const y1 = tr.y + (int64_t)(2 * g + 1) * tr.ldy + row;
            if (2 * g < NC) *y0 = (accumulate ? *y0 : 0.f) + __builtin_amdgcn_ldexpf(r0, ye0);
            if (2 * g + 1 < NC) *y1 = (accumulate ? *y1 : 0.f) + __builtin_amdgcn_ldexpf(r1, ye1);
        }
    };

    TileCursor out_cur;
    cursor_init(grp, t0v, out_cur, first.tile);
    TileRef tr_out = cursor_tile<kMvTile>(grp, t0v, out_cur, first.tile);   // matrix and rows of the tile being computed
    auto compute_and_store = [&](Item it) {
        const int sb = min(SB, nb - it.st * SB);
        const half8_t *ax = lds_x + (it.st * SB * 2 * 4) * NR + arow;
        // first half of the stage, then the second unless the stage is a half one
#pragma unroll
        for (int pp = 0; pp < SB / 4; ++pp)
            mv_block_pair<NC>(lw_row + 36 * pp, ax + (2 * pp) * 2 * 4 * NR, g, sel, pm, acc0, acc1);
        if (sb == SB) {
#pragma unroll
            for (int pp = SB / 4; pp < SB / 2; ++pp)
                mv_block_pair<NC>(lw_row + 36 * pp, ax + (2 * pp) * 2 * 4 * NR, g, sel, pm, acc0, acc1);
        }
        if (it.st == ns - 1) {
            const float r0 = acc0[0] + acc1[0], r1 = acc0[1] + acc1[1];
            if (it.tile == first.tile && first.st != 0) {
                pend = float2_t{r0, r1};
                has_pend = true;
            } else {
                store_tile(tr_out, r0, r1);
            }
            acc0[0] = acc0[1] = acc1[0] = acc1[1] = 0.f;
        }
    };

    Item cur = first;
    Item nxt = next_item(cur);

    // One stage in flight: park the stage that arrived, issue the next one into the
    // same registers, then decode the parked stage -- its decode takes several times
    // the memory latency, and the registers saved buy a fifth wave per SIMD.  A plain
    // counted loop with no exit in the middle, which keeps the compiler's wait counts
    // exact.  (The step is written out rather than as a lambda over a register-array
    // reference, which the compiler would otherwise keep in scratch.)
    for (int k = 0; k < n_items; ++k) {
        Q2_0_PARK(reg)
        __builtin_amdgcn_wave_barrier();
        if (k + 1 < n_items) Q2_0_ISSUE(nxt, reg)   // nothing after the last item: its wave ends sooner
        compute_and_store(cur);
        __builtin_amdgcn_wave_barrier();
        if (k + 1 < n_items && nxt.tile != cur.tile) tr_out = cursor_tile<kMvTile>(grp, t0v, out_cur, nxt.tile);
        cur = nxt;
        nxt = next_item(nxt);
    }
#undef Q2_0_PARK
#undef Q2_0_ISSUE
#undef Q2_0_SET_LOAD_TILE

    // An unfinished last tile leaves its partial sums for the wave that holds the
    // tile's last stage; that wave adds the earlier waves' partials in order.
    const int64_t last_tile = div_floor(i1 - 1, ns);
    const bool open_end = n_items > 0 && (i1 - 1 - last_tile * ns != ns - 1);
    if (open_end) lds_part[wave * 64 + lane] = float2_t{acc0[0] + acc1[0], acc0[1] + acc1[1]};
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
        store_tile(tile_ref<kMvTile>(grp, t0v, first.tile), r0 + pend.x, r1 + pend.y);
    }
}

// Dynamic LDS of one workgroup of `waves` waves: the wave tiles (with their dummy
// park slots), the waves' partial-tile slots and the staged activation.  Its static
// LDS (column exponents, their reduction, the partial-tile ids; under
// kMvStreamStaticLds bytes) comes on top.
size_t mat_vec_stream_lds(int N, int nb, int waves) {
    constexpr int nchunk = kMvTile * kMvStreamSB * kBlockBytes / 16;
    constexpr int dummy = (64 - (nchunk - 64 * ((nchunk + 63) / 64 - 1))) * 16;
    return (size_t)waves * (kMvTile * (kMvStreamSB * kBlockBytes + 16) + dummy + 64 * 8) +
           (size_t)nb * 2 * 4 * 2 * N * 16;
}

// Workgroup size: the wave count (4..16) that keeps the most waves resident per CU,
// given the LDS each workgroup needs (the staged activation is per workgroup) and
// the waves per SIMD the kernel's registers allow; ties go to fewer, larger groups.
// 0 if even 4 waves do not fit; *resident (optional) receives the waves per CU.
int mat_vec_stream_waves(int N, int nb, int *resident) {
    const int per_simd = 4;   // the kernel's registers allow four waves per SIMD
    int best = 0, best_res = 0;
    for (int w = kMvStreamMaxWaves; w >= 4; --w) {
        const size_t lds = mat_vec_stream_lds(N, nb, w) + kMvStreamStaticLds;
        if (lds > 160 * 1024) continue;
        int wgs = (int)((160 * 1024) / lds);
        while (wgs > 0 && wgs * w > 4 * per_simd) --wgs;
        if (wgs * w > best_res) { best_res = wgs * w; best = w; }
    }
    if (resident) *resident = best_res;
    return best;
}

template <int NC, typename XT>
static hipError_t launch_stream_nc(const MvGroup &grp, int nb, const XT *x, int64_t ldx, uint32_t rowstride,
                                   int accumulate, hipStream_t s, int grid, int waves) {
    constexpr int SB = kMvStreamSB;
    const size_t lds = mat_vec_stream_lds(NC, nb, waves);
    auto kern = mat_vec_stream<NC, SB, XT>;
    // Raise the dynamic-LDS cap once per device.  Setting it is idempotent, so threads
    // that race past the flag set the same value; the flag itself is atomic.
    static std::atomic<bool> configured[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64 || !configured[dev].load(std::memory_order_acquire)) {
        // the cap on dynamic LDS is what the kernel's static LDS leaves of 160 KiB
        hipFuncAttributes fa;
        e = hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(kern));
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)(160 * 1024 - fa.sharedSizeBytes));
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) configured[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * waves), lds, s, grp, nb, x, ldx, rowstride, accumulate);
    return hipGetLastError();
}

hipError_t launch_mat_vec_stream(const MvGroup &grp, int nb, const void *xv, Act xt, int64_t ldx, int N,
                                 hipStream_t s, uint32_t rowstride, int accumulate) {
    if (rowstride == 0) rowstride = (uint32_t)nb * kBlockBytes;
    int waves = mat_vec_stream_waves(N, nb, nullptr);
    if (waves == 0) return hipErrorInvalidValue;
    // Small launches: fewer waves per workgroup until there is a workgroup per CU.
    const int64_t ns = (nb + kMvStreamSB - 1) / kMvStreamSB;
    const int64_t items = (int64_t)grp.total_tiles * ns;
    while (waves > 4 && (items + waves - 1) / waves < 256) waves = (waves + 1) / 2 < 4 ? 4 : (waves + 1) / 2;
    const size_t lds = mat_vec_stream_lds(N, nb, waves) + kMvStreamStaticLds;
    const int per_cu = (int)((160 * 1024) / lds);
    const int max_grid = 256 * (per_cu < 1 ? 1 : per_cu);
    // every wave gets at least about one stage; never more workgroups than tiles
    int64_t need = (items + waves - 1) / waves;
    if (need > grp.total_tiles) need = grp.total_tiles;
    const int grid = (int)(need < max_grid ? need : max_grid);
    return with_act(xt, [&](auto tag) -> hipError_t {
        using XT = decltype(tag);
        const XT *x = static_cast<const XT *>(xv);
        switch (N) {
            case 1: return launch_stream_nc<1>(grp, nb, x, ldx, rowstride, accumulate, s, grid, waves);
            case 2: return launch_stream_nc<2>(grp, nb, x, ldx, rowstride, accumulate, s, grid, waves);
            case 3: return launch_stream_nc<3>(grp, nb, x, ldx, rowstride, accumulate, s, grid, waves);
            case 4: return launch_stream_nc<4>(grp, nb, x, ldx, rowstride, accumulate, s, grid, waves);
            case 5: return launch_stream_nc<5>(grp, nb, x, ldx, rowstride, accumulate, s, grid, waves);
            case 6: return launch_stream_nc<6>(grp, nb, x, ldx, rowstride, accumulate, s, grid, waves);
            case 7: return launch_stream_nc<7>(grp, nb, x, ldx, rowstride, accumulate, s, grid, waves);
            case 8: return launch_stream_nc<8>(grp, nb, x, ldx, rowstride, accumulate, s, grid, waves);
            default: return hipErrorInvalidValue;
        }
    });
}

// Blocks per chunk for a K whose activation does not fit: the largest multiple of 16
// blocks that still leaves 8 or more waves resident per CU, evened out over the chunks
// it takes; 0 if even one stage does not.  (Fewer, longer launches: at N = 8 and K =
// 6144, two chunks of 48 blocks at 8 waves per CU took 84 us for 198 MB where three of
// 32 at 16 waves took 92.)
int mat_vec_stream_chunk_blocks(int N, int nb) {
    int cb = nb / kMvStreamSB * kMvStreamSB;
    for (; cb >= kMvStreamSB; cb -= kMvStreamSB) {
        int resident = 0;
        if (mat_vec_stream_waves(N, cb, &resident) > 0 && resident >= 8) break;
    }
    if (cb < kMvStreamSB) return 0;
    const int chunks = (nb + cb - 1) / cb;
    const int even = (nb + chunks - 1) / chunks;
    return (even + kMvStreamSB - 1) / kMvStreamSB * kMvStreamSB;
}

hipError_t launch_mat_vec_stream_chunked(const MvGroup &grp, int nb, const void *xv, Act xt, int64_t ldx, int N,
                                         hipStream_t s) {
    int resident = 0;
    if (mat_vec_stream_waves(N, nb, &resident) > 0 && resident >= 8)
        return launch_mat_vec_stream(grp, nb, xv, xt, ldx, N, s, 0, 0);
    const int cb = mat_vec_stream_chunk_blocks(N, nb);
    if (cb == 0) return hipErrorInvalidValue;
    const uint32_t rowstride = (uint32_t)nb * kBlockBytes;
    for (int c0 = 0; c0 < nb; c0 += cb) {
        MvGroup g = grp;
        for (int i = 0; i < g.n; ++i) g.p[i].w += (size_t)c0 * kBlockBytes;
        const void *xc = static_cast<const uint8_t *>(xv) + (size_t)c0 * kBlockWeights * act_bytes(xt);
        const hipError_t e = launch_mat_vec_stream(g, std::min(cb, nb - c0), xc, xt, ldx, N, s, rowstride, c0 > 0);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q2_0
