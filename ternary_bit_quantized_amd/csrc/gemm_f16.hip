// Prefill GEMM on the gfx950 matrix cores: y[n][m] = sum_k W[m][k] x[n][k] with W in
// Q2_0, x rounded to fp16, f32 accumulation.
//
// bisque.today "WebGPU: add Q2_0 support", the paragraph on its three shaders: its
// tiled GEMM expands the codes to fp16 weights in workgroup memory, sixteen per
// thread, and multiplies from there.  Here no fp16 copy of W is
// made: every wave owns whole rows of the tile and unpacks them straight into its MFMA
// A operands as fp16 d*(q-1) -- exact, because d is a half and |q-1| <= 2 -- using the
// fp16-pair decode of the mat-vec (OR the code under a magic exponent, one packed
// subtract) and one packed multiply by d.  Only the raw code bytes pass through LDS
// (a wave-private area), and only x is shared between the waves.
//
//  * x is converted once per call into the caller's workspace as fp16, each column
//    scaled by a power of two that keeps it inside fp16's normal range (undone on
//    the results), and within every group of 16 k its order is permuted to (0, 8,
//    1, 9, ..., 7, 15): the order in which the pair decode emits a word's 16
//    weights.  A and B then share the k order without any shuffling.
//  * Workgroup tile (128 RF) (m) x 128 (n), four waves of (32 RF) x 128, each an RF x 4
//    grid of v_mfma_f32_32x32x16_f16; one Q2_0 block (64 k) per step.
//  * x tiles go straight from global memory to LDS (LDS-DMA), loaded one or two steps
//    ahead; one barrier per step.
//  * Without a K split, tiles are ordered so that all workgroups on one XCD (dispatch
//    is round-robin over the 8 XCDs) share one 128-column slice of x, which then stays
//    in that XCD's L2.
//  * A launch may cover several matrices that share K and x (q/k/v, gate/up): their
//    row tiles are numbered across the group and x is converted once for all.
//  * The tile height and the K split (at most 8 ways) come from a model of the busiest
//    CU's time; every split writes its partial tile to the workspace and a reduction
//    kernel adds them in split order (deterministic).  Finishing the tile in the last
//    split to arrive would save that launch, but the partials cross XCDs whose L2 caches
//    are not coherent: device-scope stores bypass the write-back L2 and L2 flushes stall
//    every workgroup, and both measured several times slower than the extra launch.
#include <climits>

#include "q2_0_internal.h"
#include "mat_vec_common.h"
#include "x_to_f16.h"

namespace q2_0 {

namespace {

constexpr int GM = 128, GK = 64;   // GM: row tile of the expert path

// One workgroup per column.  HL: the hi/lo pair of every element, the low halves lo_off
// halves after the high ones.
template <bool kVec, typename XT, bool HL = false>
__global__ __launch_bounds__(256) void x_to_f16_perm(const XT *__restrict__ x, int64_t ldx, int K,
                                                     _Float16 *__restrict__ x16, int *__restrict__ xe,
                                                     XGather gather, int64_t lo_off) {
    __shared__ float red[4];
    convert_column<kVec, XT, HL>(true, x, ldx, K, x16, xe, gather, lo_off, blockIdx.x, threadIdx.x, red);
}

// ---- W staging.  Each wave owns 32*RF rows of the tile (RF = 1 or 2 row fragments) and
// decodes them itself, straight into its MFMA A operands; no fp16 copy of W passes
// through LDS.  Per group of four blocks (72 bytes of a row) lane (rr, hf) of the wave
// loads block pair hf of its rows rr + 32i (36 bytes each, three 12-byte loads: 128 rows
// x 72 bytes take 3 coalesced loads per thread where one 2-byte load per scale and
// half-word took 24), regroups them, and writes them to
// the wave's raw area: per row 80 bytes, the four blocks' 4 code words each (an even
// block's words straddle dwords and are realigned with one v_perm), then the four
// scales, each as a half pair (d, d).  The area is private to the wave, so LDS program
// order alone orders its writes and reads (no barrier).
constexpr int kWRowDw = 20;                   // raw-area dwords per row (80 bytes)

// Raw bytes of one block pair (9 dwords: two 16-byte pieces and a last dword, the form
// the loads take, so that loop-carried copies stay in the load's register tuples) at
// byte off of a row of rowbytes bytes.  kAligned (rows of an even number of blocks from
// a 4-byte-aligned matrix): three loads, the pair's offset clamped to the row's last 36
// bytes.  Otherwise 2-byte loads, each clamped to the row's last two bytes.  Either way
// the loads stay inside the row; data past the split's blocks is never used.  (Three
// loads per pair at least: the kernel's wait counts rely on that lower bound.)
struct RawPair {
    u32x4_t a, b;   // dwords 0..3, 4..7
    uint32_t c;     // dword 8
};
template <bool kAligned>
__device__ __forceinline__ void load_pair(const uint8_t *row, int off, int rowbytes, RawPair &r) {
    if constexpr (kAligned) {
        typedef uint32_t u32x4a4_t __attribute__((ext_vector_type(4), aligned(4)));
        const uint8_t *p = row + min(off, rowbytes - 36);
        r.a = *reinterpret_cast<const u32x4a4_t *>(p);
        r.b = *reinterpret_cast<const u32x4a4_t *>(p + 16);
        r.c = *reinterpret_cast<const uint32_t *>(p + 32);
    } else {
        const uint16_t *h = reinterpret_cast<const uint16_t *>(row);
        const int lim = (rowbytes >> 1) - 1;
        const int o = off >> 1;
        uint32_t t[9];
#pragma unroll
        for (int i = 0; i < 9; ++i)
            t[i] = (uint32_t)h[min(o + 2 * i, lim)] | ((uint32_t)h[min(o + 2 * i + 1, lim)] << 16);
        r.a = u32x4_t{t[0], t[1], t[2], t[3]};
        r.b = u32x4_t{t[4], t[5], t[6], t[7]};
        r.c = t[8];
    }
}

}  // namespace

// One launch's matrices (see GemmGroup in q2_0_internal.h): row tiles are numbered
// across the whole call; tm0 repeats the items' first row tiles contiguously (entries
// past n hold INT_MAX) for a binary-search lookup.
__device__ __forceinline__ int find_gemm_item(const GemmGroup &grp, int tmg) {
    int idx = 0;
#pragma unroll
    for (int step = kGemmMaxGroup / 2; step >= 1; step >>= 1)
        if (grp.tm0[idx + step] <= tmg) idx += step;
    return idx;
}

// splits > 1: workgroup (tile, split) covers blocks [split*nbs, (split+1)*nbs) and writes
// its partial tile to the item's part + split*N*M (column n at n*M); gemm_split_reduce
// then adds the partials in split order.
// Steps run in groups of four blocks; the steps of a split's last group past its end
// load (clamped) like the others but skip the decode and the MFMAs.  The workgroup tile
// is (128 RF) x 128: four waves of (32 RF) x 128.
//
// x tiles go global -> LDS directly (16-byte LDS-DMA loads: lane i of a wave's load
// lands at the destination + 16 i), NXB LDS buffers, each step's tile loaded NXB - 1
// steps ahead.  A column's 64 k (128 bytes, 8 chunks of 16) sit unpadded, chunk ch of column c
// at position ch ^ ((c >> 1) & 7): a 16-byte operand read is served 16 lanes at a time
// across the 64 banks, and the 16 consecutive columns of such a group (one chunk each)
// then fall on 16 distinct 16-byte bank groups (an even and an odd column share no
// group, and the 8 even or odd ones differ in c >> 1); a load lane picks the global chunk
// that belongs at its LDS position.  (With ch ^ (c & 7) the groups of 16 met in pairs:
// ~7x the bank-conflict cycles, measured.)
// One 16-byte LDS-DMA load per lane: lane i's 16 bytes at src land at LDS byte address
// lds + 16 i.  Issued as inline assembly so that the compiler does not track it: its
// own wait insertion would otherwise make every later LDS read wait for all of these
// loads (it cannot tell that they fill a different buffer).  The caller orders them
// with wait_vmcnt before the barrier that publishes the tile.
// M0 (the LDS address) is saved and restored around the load, so the compiler's view of
// it does not change.
__device__ __forceinline__ void lds_dma16(const void *src, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(lds)
        : "memory");
}

// s_waitcnt with only the vector-memory count set (expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int RF, int NJ, int NXB, bool kAligned, int OCC, bool HL>
__global__ __launch_bounds__(256, OCC) void gemm_f16_mfma(GemmGroup grp, int nb, const _Float16 *__restrict__ x16,
                                                          const int *__restrict__ xe, int N, int tiles_n,
                                                          int xcd_map, int splits, int64_t lo_off) {
    static_assert(RF == 1 || RF == 2, "one or two row fragments per wave");
    static_assert(NJ == 2 || NJ == 4, "two or four column fragments per wave");
    static_assert(NXB == 2 || NXB == 3, "two or three x buffers");
    static_assert(!HL || NXB == 2, "hi/lo: two x buffers");
    constexpr int TM = 128 * RF, TN = 32 * NJ, kWRows = 32 * RF, kWAreaDw = kWRows * kWRowDw;
    constexpr int BSZ = (HL ? 2 : 1) * TN * GK;   // a buffer: the x tile (HL: its hi, then its lo halves)
    __shared__ __attribute__((aligned(16))) _Float16 Bs[NXB][BSZ];
    __shared__ __attribute__((aligned(16))) uint32_t Wraw[4 * kWAreaDw];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // ---- tile of this workgroup (row tile tmg counted across the call).  xcd_map: XCD
    // j = blockIdx % 8 handles column tile j % tiles_n and every (8 / tiles_n)-th row tile.
    int tl, tn;
    const int split = blockIdx.x % splits;
    {
        const int b = blockIdx.x / splits;
        if (xcd_map) {
            const int j = b & 7, l = b >> 3;
            const int per = 8 / tiles_n;     // XCDs per column tile
            tn = j % tiles_n;
            tl = l * per + j / tiles_n;
        } else {
            tn = b % tiles_n;
            tl = b / tiles_n;
        }
    }
    // matrix, rows and columns of this workgroup's tile: all N columns of the call, or
    // (expert routing) a column tile of one expert's own run of x16
    const uint8_t *__restrict__ w;
    int M, m0, n0, col0 = 0, Nv = N;
    const GemmItem *itp;
    if (!grp.moe_off) {
        const int tmg = grp.tm_base + tl;
        itp = &grp.p[find_gemm_item(grp, tmg)];
        w = itp->w;
        M = itp->M;
        m0 = (tmg - itp->tm0) * TM;
        n0 = tn * TN;
    } else {
        const int t = blockIdx.x / grp.moe_tiles_m;
        if (t >= grp.moe_max_tiles) {       // NaN into the out-of-range pairs' columns
            const GemmItem &it = grp.p[0];
            const int m = (blockIdx.x % grp.moe_tiles_m) * TM + (tid % TM);
            const int j1 = grp.moe_off[grp.moe_n_expert + 1];
            if (m < it.M)
                for (int j = grp.moe_off[grp.moe_n_expert] + tid / TM; j < j1; j += 256 / TM)
                    it.y[(int64_t)grp.moe_perm[j] * it.ldy + m] = __builtin_nanf("");
            return;
        }
        if (t >= *grp.moe_ntiles) return;   // the whole workgroup: no tile here
        const int e = grp.moe_tiles[2 * t];
        itp = &grp.p[0];
        w = itp->w + e * grp.moe_expert_bytes;
        M = itp->M;
        m0 = (blockIdx.x % grp.moe_tiles_m) * TM;
        n0 = grp.moe_tiles[2 * t + 1] * TN;
        col0 = grp.moe_off[e];
        Nv = grp.moe_off[e + 1] - col0;
    }
    const GemmItem &item = *itp;
    // x16 row of column n of the tile (columns past Nv use the tile's first column)
    auto xrow = [&](int n) {
        const int c = col0 + (n < Nv ? n : 0);
        return grp.moe_off ? grp.moe_perm[c] / grp.moe_xdiv : c;
    };
    const int K = nb * kBlockWeights;
    const int rowbytes = nb * kBlockBytes;
    const int nbs = nb / splits;                 // blocks of this split
    const int kb0 = split * nbs;
    const int ngroups = (nbs + 3) >> 2;

    // ---- W loader: lane (rr, hf) = block pair hf of rows rr + 32i of this wave's rows.  Rows
    // past M read row M-1 (they feed outputs that are never stored); byte offsets are
    // clamped to the row's last 36 bytes, so a padded group stays inside the matrix.
    const int wrow0 = m0 + kWRows * wave;
    const int rbase = min(wrow0, M - 1);
    const uint8_t *const wbase = w + (int64_t)rbase * rowbytes;
    const int rr = lane >> 1, hf = lane & 1;
    uint32_t roff[RF];
#pragma unroll
    for (int i = 0; i < RF; ++i) roff[i] = (uint32_t)(min(wrow0 + rr + 32 * i, M - 1) - rbase) * (uint32_t)rowbytes;
    auto load_raw = [&](int grp4, RawPair (&r)[RF]) {
#pragma unroll
        for (int i = 0; i < RF; ++i)
            load_pair<kAligned>(wbase + roff[i], (kb0 + 4 * grp4 + 2 * hf) * kBlockBytes, rowbytes, r[i]);
    };
    uint32_t *const warea = Wraw + wave * kWAreaDw;
    auto write_raw = [&](int grp4, const RawPair (&rs)[RF]) {
        const int blk = 4 * grp4 + 2 * hf;       // even block of this pair, within the split
#pragma unroll
        for (int i = 0; i < RF; ++i) {
            const RawPair &r = rs[i];
            u32x4_t ev, od;
            ev.x = __builtin_amdgcn_perm(r.a.y, r.a.x, 0x05040302u);
            ev.y = __builtin_amdgcn_perm(r.a.z, r.a.y, 0x05040302u);
            ev.z = __builtin_amdgcn_perm(r.a.w, r.a.z, 0x05040302u);
            ev.w = __builtin_amdgcn_perm(r.b.x, r.a.w, 0x05040302u);
            od = u32x4_t{r.b.y, r.b.z, r.b.w, r.c};
            const uint32_t de = blk < nbs ? __builtin_amdgcn_perm(r.a.x, r.a.x, 0x01000100u) : 0u;
            const uint32_t dod = blk + 1 < nbs ? __builtin_amdgcn_perm(r.b.x, r.b.x, 0x03020302u) : 0u;
            uint32_t *row = warea + (rr + 32 * i) * kWRowDw;
            *reinterpret_cast<u32x4_t *>(row + 8 * hf) = ev;
            *reinterpret_cast<u32x4_t *>(row + 8 * hf + 4) = od;
            *reinterpret_cast<u32x2_t *>(row + 16 + 2 * hf) = u32x2_t{de, dod};
        }
    };

    // ---- x loader: wave w fills columns 8NJ w .. 8NJ (w+1) - 1 of a tile, NJ LDS-DMA loads
    // of 8 columns; lane i: column c = 8NJ w + 8q + i/8, LDS chunk position i%8, global
    // chunk (i%8) ^ ((c >> 1) & 7) (= (i%8) ^ (i/16 + 4 (q & 1)), NJ being even).  Columns
    // past N read column 0 (outputs never stored); blocks past the split are clamped to its
    // last block (loaded but never multiplied).
    const _Float16 *xsrc[NJ];
    {
        const int cq = lane >> 3;
#pragma unroll
        for (int q = 0; q < NJ; ++q) {
            const int n = n0 + 8 * NJ * wave + 8 * q + cq;
            const int ch = (lane & 7) ^ ((cq >> 1) | ((q & 1) << 2));
            xsrc[q] = x16 + (int64_t)xrow(n) * K + (int64_t)kb0 * GK + 8 * ch;
        }
    }
    const uint32_t bs_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)&Bs[0][0];
    auto load_x = [&](int buf, int blk) {
        blk = min(blk, nbs - 1);
        const uint32_t dst = __builtin_amdgcn_readfirstlane(bs_lds + (uint32_t)(buf * BSZ + 8 * NJ * wave * GK) * 2u);
#pragma unroll
        for (int q = 0; q < NJ; ++q) lds_dma16(xsrc[q] + (int64_t)blk * GK, dst + (uint32_t)(8 * q * GK * 2));
        if (HL) {
#pragma unroll
            for (int q = 0; q < NJ; ++q)
                lds_dma16(xsrc[q] + lo_off + (int64_t)blk * GK, dst + (uint32_t)((TN * GK + 8 * q * GK) * 2));
        }
    };

    float16_t acc[RF][NJ];
#pragma unroll
    for (int i = 0; i < RF; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = float16_t{};
    // HL: acc holds two blocks' sums (hi and lo products, from zero); mst adds them in
    // fp64
    double mst[HL ? RF : 1][HL ? NJ : 1][16];
#pragma unroll
    for (int i = 0; i < (HL ? RF : 1); ++i)
#pragma unroll
        for (int j = 0; j < (HL ? NJ : 1); ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) mst[i][j][v] = 0.0;

    // A lane l: row l%32 of a row fragment, k-slot (l/32)*8 of each 16-k step: word kk of
    // the block, code pairs 4h..4h+3 (h = l/32; the word is shifted down 8h bits so that
    // they sit at pairs 0..3).  In the permuted k order of x16 these are exactly the 8 k
    // that B lane (column, h) holds.  B lane: column l%32 of a 32-column sub-tile.
    const int frow = lane & 31;
    const uint32_t sh = (uint32_t)(lane >> 5) * 8u;
    int bsw[4];   // swizzled position (halves) of chunk 2kk + h of this lane's columns
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) bsw[kk] = 8 * ((2 * kk + (lane >> 5)) ^ ((frow >> 1) & 7));
    const PairMasks pm;
    const uint32_t *const wmy = warea + frow * kWRowDw;
    struct WStep {
        u32x4_t wd[RF];   // the block's 4 code words, per row fragment
        half2_t dd[RF];   // its scale pair
    };
    auto read_w = [&](int b) {
        WStep r;
#pragma unroll
        for (int i = 0; i < RF; ++i) {
            r.wd[i] = *reinterpret_cast<const u32x4_t *>(wmy + 32 * i * kWRowDw + 4 * b);
            r.dd[i] = __builtin_bit_cast(half2_t, wmy[32 * i * kWRowDw + 16 + b]);
        }
        return r;
    };
    // Column fragments with a live column (uniform); in the expert product's configuration
    // (NJ = 2 without hi/lo: its tiles are often part empty) the others skip their operand
    // reads and products (128 experts of 768 x 2048 at 128 tokens: 40.8 -> 35.5 us per
    // call).  The dense configurations keep every product: their tiles are full, and the
    // branches measured 6-10 % slower on the prefill.
    constexpr bool kSkipEmpty = NJ == 2 && !HL;
    bool live[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) live[j] = !kSkipEmpty || n0 + 32 * j < Nv;
    auto step = [&](int buf, const WStep &ws) {
        const u32x4_t *wd = ws.wd;
        const half2_t *dd = ws.dd;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            half8_t a[RF];
#pragma unroll
            for (int i = 0; i < RF; ++i) {
                const uint32_t c = wd[i][kk] >> sh;
                const half2_t d2 = dd[i];
                a[i] = as_half8(__builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, pair_qm1<0>(c, pm)) * d2),
                                __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, pair_qm1<1>(c, pm)) * d2),
                                __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, pair_qm1<2>(c, pm)) * d2),
                                __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, pair_qm1<3>(c, pm)) * d2));
            }
            half8_t bv[NJ], bl[HL ? NJ : 1];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if (kSkipEmpty && j > 0 && !live[j]) continue;
                bv[j] = *reinterpret_cast<const half8_t *>(&Bs[buf][(j * 32 + frow) * GK + bsw[kk]]);
                if (HL) bl[j] = *reinterpret_cast<const half8_t *>(&Bs[buf][TN * GK + (j * 32 + frow) * GK + bsw[kk]]);
            }
#pragma unroll
            for (int i = 0; i < RF; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    if (kSkipEmpty && j > 0 && !live[j]) continue;
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], bv[j], acc[i][j], 0, 0, 0);
                    if (HL) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], bl[HL ? j : 0], acc[i][j], 0, 0, 0);
                }
        }
    };
    // HL: every two blocks the f32 sums go into the fp64 ones and start again from zero
    auto flush = [&]() {
        if constexpr (HL) {
#pragma unroll
            for (int i = 0; i < RF; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) mst[i][j][v] += (double)acc[i][j][v];
                    acc[i][j] = float16_t{};
                }
        }
    };

    // ---- pipeline.  Step t multiplies x buffer t % NXB while the tile of step t+NXB-1
    // loads into buffer (t+NXB-1) % NXB (last read at step t-1, before the barrier that
    // ended it).  W raw groups are loaded one group ahead into registers; a group's last
    // step reads its own words first, then writes the next group to the wave's area and
    // issues the loads of the one after, and the x load, then the MFMAs.  Before the
    // barrier that ends step t each wave waits for its own loads of tile t+1; younger are
    // (NXB = 3) tile t+2's four and, in a group's last step, the raw loads issued before
    // them; (NXB = 2) in a group's last step the raw loads, issued after the tile so that
    // they stay in flight into the next step (whose wait, for a younger tile, ends them),
    // otherwise none.  Raw loads are counted per row fragment as three 12-byte loads (at
    // least that many are issued); the 2-byte path counts none (its waits then also
    // cover them).
    constexpr int kRaw = kAligned ? 3 * RF : 0;
    RawPair wr[RF];
    load_raw(0, wr);
#pragma unroll
    for (int i = 0; i + 1 < NXB; ++i) load_x(i, i);
    write_raw(0, wr);
    load_raw(1, wr);
    wait_vmcnt<kRaw>();          // x tiles 0 .. NXB-2 (younger: raw group 1)
    __syncthreads();

    int buf = 0;                 // t % NXB
    for (int g = 0; g < ngroups; ++g) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = 4 * g + u;
            const int bufn = NXB == 3 ? (buf == 0 ? 2 : buf - 1) : (buf ^ 1);   // (t + NXB - 1) % NXB
            const WStep ws = read_w(u);
            if (u == 3) write_raw(g + 1, wr);   // after this step's read of the area
            if constexpr (NXB == 3) {
                if (u == 3) load_raw(g + 2, wr);
                load_x(bufn, t + NXB - 1);
            } else {
                // two x buffers: the raw loads go out after the x tile, so that the wait
                // for the tile leaves them in flight until the next step's wait
                load_x(bufn, t + NXB - 1);
                if (u == 3) load_raw(g + 2, wr);
            }
            if (t < nbs) step(buf, ws);
            if (HL && (u & 1)) flush();
            if constexpr (NXB == 3) {
                if (u == 3)
                    wait_vmcnt<NJ + kRaw>();   // tile t+1 (younger: raw group g+2, tile t+2)
                else
                    wait_vmcnt<NJ>();          // tile t+1 (younger: tile t+2)
            } else {
                if (u == 3)
                    wait_vmcnt<kRaw>();       // tile t+1 (younger: raw group g+2)
                else
                    wait_vmcnt<0>();          // tile t+1 (issued last; older raw loads with it)
            }
            __syncthreads();
            buf = NXB == 3 ? (buf == 2 ? 0 : buf + 1) : (buf ^ 1);
        }
    }

    // ---- epilogue: D lane l, register v -> row 8*(v/4) + 4*(l/32) + v%4, column l%32
    // Results are scaled back by the column's 2^-e first (exact), so partials and y
    // hold the same numbers.
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int n = n0 + j * 32 + (lane & 31);
        const int ye = -xe[xrow(n)];
#pragma unroll
        for (int i = 0; i < RF; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                if constexpr (HL)
                    acc[i][j][v] = (float)__builtin_amdgcn_ldexp(mst[HL ? i : 0][HL ? j : 0][v], ye);   // one rounding
                else
                    acc[i][j][v] = __builtin_amdgcn_ldexpf(acc[i][j][v], ye);
            }
    }
    // Stores of a 4-row run of column n at row m: float4 when in range and aligned.
    auto store4 = [&](float *col, int m, const float4_t &val) {
        if (m + 3 < M && ((((uintptr_t)(col + m)) & 15) == 0)) {
            *reinterpret_cast<float4_t *>(col + m) = val;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (m + e < M) col[m + e] = val[e];
        }
    };
    // With a K split the tile goes to this split's partial (summed by gemm_split_reduce).
    float *const yout = (splits > 1) ? item.part + (int64_t)split * N * M : item.y;
    const int64_t ldo = (splits > 1) ? M : item.ldy;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int n = n0 + j * 32 + (lane & 31);
        if (n >= Nv) continue;
        float *yc = grp.moe_off ? item.y + (int64_t)grp.moe_perm[col0 + n] * item.ldy : yout + (int64_t)n * ldo;
#pragma unroll
        for (int i = 0; i < RF; ++i)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int m = wrow0 + 32 * i + 8 * v4 + 4 * (lane >> 5);
                store4(yc, m, float4_t{acc[i][j][4 * v4], acc[i][j][4 * v4 + 1], acc[i][j][4 * v4 + 2],
                                       acc[i][j][4 * v4 + 3]});
            }
    }
}

// y_i[n][m] = sum over splits of part_i[split][n][m], in split order.  Grid: x over
// 1024-row chunks of a column, y over the N columns (strided past 65535), z over the
// launch's matrices;
// each thread adds four consecutive rows (16-byte accesses when aligned).
__global__ __launch_bounds__(256) void gemm_split_reduce(GemmGroup grp, int splits, int N) {
    const GemmItem &it = grp.p[blockIdx.z];
    const int M = it.M;
    const int m = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (m >= M) return;
    const int64_t per = (int64_t)N * M;
    for (int n = blockIdx.y; n < N; n += gridDim.y) {
        const float *src = it.part + (int64_t)n * M + m;
        float *dst = it.y + (int64_t)n * it.ldy + m;
        const bool vec = m + 3 < M && (((uintptr_t)src | (uintptr_t)dst) & 15) == 0 && (M & 3) == 0;
        if (vec) {
            float4_t acc = *reinterpret_cast<const float4_t *>(src);
            for (int sp = 1; sp < splits; ++sp) acc += *reinterpret_cast<const float4_t *>(src + sp * per);
            *reinterpret_cast<float4_t *>(dst) = acc;
        } else {
            for (int e = 0; e < 4 && m + e < M; ++e) {
                float acc = src[e];
                for (int sp = 1; sp < splits; ++sp) acc += src[e + sp * per];
                dst[e] = acc;
            }
        }
    }
}

namespace {

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

// GEMM kernel configurations (workgroup tile rows x columns, per wave RF x NJ MFMA tiles):
//   A: 128 x 128, RF 1 x NJ 4, two x buffers, three workgroups per CU;
//   B: 256 x 128, RF 2 x NJ 4, three x buffers, two workgroups per CU.
//   C: 128 x 64, RF 1 x NJ 2, two x buffers, four workgroups per CU: the expert product,
//      whose experts hold a few dozen columns each (half the MFMAs and x loads of A per
//      tile there, for the same weight decode).
//   D: C's tile with x as hi/lo pairs (fp32-grade): two x tiles per buffer, two MFMAs
//      per operand pair (so each decoded weight fragment feeds four, as in A), an f32
//      accumulator per two blocks and the fp64 sums in registers; two workgroups per CU (at three the registers spill; A's
//      128-column tile would need 128 registers of fp64 sums per lane and spills too).
// (256 x 64 tiles, RF 2 x NJ 2 at three workgroups per CU -- half the LDS operand reads
// per MFMA of A, twice the decode per MFMA -- measured ~10 % slower than A at N = 512.)
enum GemmCfg { kCfgA = 0, kCfgB = 1, kCfgC = 2, kCfgD = 3 };
constexpr int cfg_rows(int cfg) { return cfg == kCfgB ? 256 : 128; }
constexpr int cfg_cols(int cfg) { return (cfg == kCfgC || cfg == kCfgD) ? 64 : 128; }

// The GEMM kernel of a configuration, with 4-byte code loads where every matrix row is
// 4-byte aligned.
// lo_off: configuration D's distance (halves) from the high to the low halves of x16.
static void launch_gemm_kernel(unsigned grid, hipStream_t s, const GemmGroup &grp, int nb, const _Float16 *x16,
                               const int *xe, int N, int tiles_n, int xcd_map, int splits, int cfg, bool aligned,
                               int64_t lo_off = 0) {
#define Q2_0_GEMM_LAUNCH(RF, NJ, NXB, OCC, HL)                                                                   \
    do {                                                                                                        \
        if (aligned)                                                                                            \
            gemm_f16_mfma<RF, NJ, NXB, true, OCC, HL><<<grid, 256, 0, s>>>(grp, nb, x16, xe, N, tiles_n,  \
                                                                                 xcd_map, splits, lo_off);     \
        else                                                                                                    \
            gemm_f16_mfma<RF, NJ, NXB, false, OCC, HL><<<grid, 256, 0, s>>>(grp, nb, x16, xe, N, tiles_n, \
                                                                                  xcd_map, splits, lo_off);    \
    } while (0)
    if (cfg == kCfgB)
        Q2_0_GEMM_LAUNCH(2, 4, 3, 2, false);
    else if (cfg == kCfgC)
        Q2_0_GEMM_LAUNCH(1, 2, 2, 4, false);
    else if (cfg == kCfgD)
        Q2_0_GEMM_LAUNCH(1, 2, 2, 2, true);
    else
        Q2_0_GEMM_LAUNCH(1, 4, 2, 3, false);
#undef Q2_0_GEMM_LAUNCH
}

// Configuration and K split of a call, from a model of the busiest CU's time.
// Workgroups go out in rounds of (workgroups per CU) x 256; a round in which a CU holds
// w of them takes (blocks per split) x step time(w).  A K split s adds its partials,
// written by the GEMM (s N M floats at ~5 TB/s) and read back with the result written
// by the reduction ((s + 1) N M floats at ~4.5 TB/s, plus its launch).  The constants
// are fitted to kernel traces of the stack's shapes at N = 512 on MI355X for every split
// (0.74, 0.60 and 0.58 us per 128-row workgroup-step with 1, 2 and 3 of them on a CU,
// the busiest CU's partial writes included).  Candidates: A with s in
// {1, 2, 3, 4, 6, 8} (s dividing the blocks, at least 8 per split and, for even block
// counts, an even number), B without a split and only for an even block count.  Ties
// keep the earlier candidate (smaller split, A).  The fp32-grade calls (hi/lo x) have D
// alone, with the same splits.
struct GemmPlan {
    int cfg, splits;
};
constexpr double kStepUs[3][4] = {
    {0.0, 0.74, 1.20, 1.75},   // A, by concurrent workgroups per CU
    {0.0, 1.00, 1.87, 0.0},    // B
    {0.0, 0.85, 1.40, 0.0},    // D
};
constexpr int kPerCu[3] = {3, 2, 2};
constexpr int cfg_row(int cfg) { return cfg == kCfgB ? 1 : cfg == kCfgD ? 2 : 0; }
constexpr double kPartWriteBytesPerUs = 5.0e6, kReduceBytesPerUs = 4.5e6, kReduceLaunchUs = 2.0;

static double rounds_us(int64_t wgs, int per_cu, const double *step_us, int steps) {
    const int64_t slots = 256 * (int64_t)per_cu;
    const int64_t full = (wgs - 1) / slots;                  // rounds before the last
    const int64_t last = wgs - full * slots;                 // workgroups in the last round
    const int w_last = (int)((last + 255) / 256);
    return ((double)full * step_us[per_cu] + step_us[w_last]) * steps;
}

static GemmPlan gemm_plan(const q2_0_mat_vec_item *items, int64_t n_items, int nb, int64_t N, bool hl) {
    int64_t rows = 0, tiles[2] = {0, 0};
    for (int64_t i = 0; i < n_items; ++i) {
        tiles[0] += (items[i].M + 127) / 128;
        tiles[1] += (items[i].M + 255) / 256;
        rows += items[i].M;
    }
    const double nm_bytes = 4.0 * (double)N * (double)rows;   // one f32 copy of all outputs
    GemmPlan best{hl ? kCfgD : kCfgA, 1};
    double best_us = 1e300;
    const int cands[2] = {hl ? kCfgD : kCfgA, kCfgB};
    for (int c = 0; c < (hl ? 1 : 2); ++c) {
        const int cfg = cands[c];
        if (cfg == kCfgB && nb % 2 != 0) continue;
        const int64_t t = tiles[cfg == kCfgB ? 1 : 0] * ((N + cfg_cols(cfg) - 1) / cfg_cols(cfg));
        for (int sp : {1, 2, 3, 4, 6, 8}) {
            if (sp > 1 && (cfg == kCfgB || nb % sp != 0 || nb / sp < 8 || (nb % 2 == 0 && (nb / sp) % 2 != 0)))
                continue;
            double us = rounds_us(t * sp, kPerCu[cfg_row(cfg)], kStepUs[cfg_row(cfg)], nb / sp);
            if (sp > 1)
                us += sp * nm_bytes / kPartWriteBytesPerUs + (sp + 1) * nm_bytes / kReduceBytesPerUs + kReduceLaunchUs;
            if (us < best_us) {
                best_us = us;
                best = {cfg, sp};
            }
        }
    }
    return best;
}

// Workspace of a call: fp16 x (N*K halves; hl: the high halves, then the low ones), the
// column exponents (N ints), and with a K split each matrix's partials (splits * N * M
// floats).
static size_t x16_bytes(int64_t N, int64_t K, bool hl) { return align256((size_t)N * K * 2 * (hl ? 2 : 1)); }

static size_t gemm_layout(const q2_0_mat_vec_item *items, int64_t n_items, int nb, int64_t N, bool hl,
                          GemmPlan *plan, size_t *parts_off) {
    const GemmPlan pl = gemm_plan(items, n_items, nb, N, hl);
    const int64_t K = (int64_t)nb * kBlockWeights;
    size_t off = x16_bytes(N, K, hl) + align256((size_t)N * 4);
    *parts_off = off;
    if (pl.splits > 1)
        for (int64_t i = 0; i < n_items; ++i) off += align256((size_t)pl.splits * N * items[i].M * 4);
    *plan = pl;
    return off;
}

size_t gemm_f16_workspace_bytes(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K, int64_t N, bool hl) {
    GemmPlan pl;
    size_t po;
    return gemm_layout(items, n_items, (int)(K / kBlockWeights), N, hl, &pl, &po);
}

int gemm_f16_splits(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K, int64_t N, bool hl) {
    return gemm_plan(items, n_items, (int)(K / kBlockWeights), N, hl).splits;
}

hipError_t launch_gemm_f16_group(const q2_0_mat_vec_item *mats, int64_t n_items, int nb, const void *x, Act xt,
                                 int64_t ldx, int64_t N, void *workspace, hipStream_t s, bool hl) {
    const int K = nb * kBlockWeights;
    GemmPlan plan;
    size_t parts_off;
    gemm_layout(mats, n_items, nb, N, hl, &plan, &parts_off);
    const int splits = plan.splits, TM = cfg_rows(plan.cfg), TN = cfg_cols(plan.cfg);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    _Float16 *x16 = reinterpret_cast<_Float16 *>(ws);
    int *xe = reinterpret_cast<int *>(ws + x16_bytes(N, K, hl));
    const int64_t lo_off = hl ? N * (int64_t)K : 0;
    const int tiles_n = (int)((N + TN - 1) / TN);

    const bool vec = ((uintptr_t)x % (4 * act_bytes(xt)) == 0) && (ldx % 4 == 0);
    hipError_t e = with_act(xt, [&](auto tag) -> hipError_t {
        using XT = decltype(tag);
        const XT *xp = static_cast<const XT *>(x);
        const XGather g{nullptr, 1, 1};
        if (vec && hl)
            x_to_f16_perm<true, XT, true><<<(unsigned)N, 256, 0, s>>>(xp, ldx, K, x16, xe, g, lo_off);
        else if (vec)
            x_to_f16_perm<true, XT><<<(unsigned)N, 256, 0, s>>>(xp, ldx, K, x16, xe, g, 0);
        else if (hl)
            x_to_f16_perm<false, XT, true><<<(unsigned)N, 256, 0, s>>>(xp, ldx, K, x16, xe, g, lo_off);
        else
            x_to_f16_perm<false, XT><<<(unsigned)N, 256, 0, s>>>(xp, ldx, K, x16, xe, g, 0);
        return hipGetLastError();
    });
    if (e != hipSuccess) return e;

    // one launch (plus one reduction with a K split) per kGemmMaxGroup matrices
    float *part = reinterpret_cast<float *>(ws + parts_off);
    int64_t tm_next = 0;
    for (int64_t i0 = 0; i0 < n_items; i0 += kGemmMaxGroup) {
        GemmGroup grp;
        grp.n = 0;
        grp.tm_base = (int)tm_next;
        grp.moe_off = nullptr;
        for (int64_t i = i0; i < n_items && i < i0 + kGemmMaxGroup; ++i) {
            const int64_t M = mats[i].M;
            if (M == 0) continue;
            GemmItem &it = grp.p[grp.n];
            it.w = static_cast<const uint8_t *>(mats[i].w);
            it.y = mats[i].y;
            it.ldy = mats[i].ldy;
            it.part = part;
            it.M = (int)M;
            it.tm0 = (int)tm_next;
            grp.tm0[grp.n] = it.tm0;
            ++grp.n;
            tm_next += (M + TM - 1) / TM;
            if (splits > 1) part += align256((size_t)splits * N * M * 4) / 4;
        }
        if (grp.n == 0) continue;
        for (int k = grp.n; k < kGemmMaxGroup; ++k) grp.tm0[k] = INT_MAX;
        const int tiles_m = (int)tm_next - grp.tm_base;
        const int per = (tiles_n <= 8 && 8 % tiles_n == 0) ? 8 / tiles_n : 0;
        const int xcd_map = (splits == 1 && per != 0 && tiles_m % per == 0) ? 1 : 0;
        bool aligned = nb % 2 == 0;
        for (int k = 0; k < grp.n; ++k) aligned = aligned && ((uintptr_t)grp.p[k].w % 4 == 0);
        launch_gemm_kernel((unsigned)(tiles_m * tiles_n * splits), s, grp, nb, x16, xe, (int)N, tiles_n, xcd_map,
                           splits, plan.cfg, aligned, lo_off);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (splits > 1) {
            int maxM = 0;
            for (int k = 0; k < grp.n; ++k) maxM = grp.p[k].M > maxM ? grp.p[k].M : maxM;
            const dim3 rgrid((unsigned)((maxM + 1023) / 1024), (unsigned)(N < 65535 ? N : 65535), (unsigned)grp.n);
            gemm_split_reduce<<<rgrid, 256, 0, s>>>(grp, splits, (int)N);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

// Expert product on the fp16 GEMM: x is converted once, one row per token (one per pair
// when every slot has its own x column; scratch: x16 then the row exponents), then one
// launch runs every (expert, column tile) entry of the routing's tile list against all
// row tiles, each column's x row read through the routing's pair index; entries past
// the list's length exit at once.  No K split, so every result is written once, in a
// fixed order.
size_t gemm_f16_moe_scratch_bytes(int64_t K, int64_t n_pairs) {
    return align256((size_t)n_pairs * K * 2) + align256((size_t)n_pairs * 4);
}

hipError_t launch_gemm_f16_moe(const uint8_t *w, int64_t M, int nb, const void *x, Act xt, int64_t ldx,
                               const MoeRoute &r, float *y, int64_t ldy, void *scratch, hipStream_t s,
                               bool x_ready) {
    const int K = nb * kBlockWeights;
    uint8_t *ws = static_cast<uint8_t *>(scratch);
    _Float16 *x16 = reinterpret_cast<_Float16 *>(ws);
    int *xe = reinterpret_cast<int *>(ws + align256((size_t)r.n_pairs * K * 2));
    if (!x_ready) {
        const bool vec = ((uintptr_t)x % (4 * act_bytes(xt)) == 0) && (ldx % 4 == 0);
        const XGather ident{nullptr, r.n_used, r.x_slots};
        const int nx = moe_x_rows(r.n_pairs, r.n_used, r.x_slots);
        hipError_t e = with_act(xt, [&](auto tag) -> hipError_t {
            using XT = decltype(tag);
            const XT *xp = static_cast<const XT *>(x);
            if (vec)
                x_to_f16_perm<true, XT><<<(unsigned)nx, 256, 0, s>>>(xp, ldx, K, x16, xe, ident, 0);
            else
                x_to_f16_perm<false, XT><<<(unsigned)nx, 256, 0, s>>>(xp, ldx, K, x16, xe, ident, 0);
            return hipGetLastError();
        });
        if (e != hipSuccess) return e;
    }
    const int tiles_m = (int)((M + GM - 1) / GM);
    GemmGroup grp;
    grp.n = 1;
    grp.tm_base = 0;
    grp.p[0] = GemmItem{w, y, ldy, nullptr, (int)M, 0};
    for (int k = 0; k < kGemmMaxGroup; ++k) grp.tm0[k] = k ? INT_MAX : 0;
    grp.moe_off = r.off;
    grp.moe_perm = r.perm;
    grp.moe_tiles = r.tiles;
    grp.moe_ntiles = r.ntiles;
    grp.moe_expert_bytes = M * (int64_t)nb * kBlockBytes;
    grp.moe_tiles_m = tiles_m;
    grp.moe_xdiv = r.x_slots == 1 ? r.n_used : 1;
    if (r.tile_w != cfg_cols(kCfgC)) return hipErrorInvalidValue;
    grp.moe_max_tiles = (int)moe_max_tiles(r.n_expert, r.n_pairs, cfg_cols(kCfgC));
    grp.moe_n_expert = r.n_expert;
    const int64_t grid = (int64_t)tiles_m * (grp.moe_max_tiles + 1);   // + the NaN fill
    launch_gemm_kernel((unsigned)grid, s, grp, nb, x16, xe, (int)r.n_pairs, 1, 0, 1, kCfgC,
                       nb % 2 == 0 && (uintptr_t)w % 4 == 0);
    return hipGetLastError();
}

}  // namespace q2_0
