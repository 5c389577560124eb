// Expert ("mixture of experts") product: y[t][u] = W_{ids[t][u]} x[t][u mod x_slots].
//
// bisque.today "WebGPU: add Q2_0 support" leaves the expert mat-mul out for Q2_0 (the
// paragraph on what the change does not cover); this is that product on the same
// block decode.  The routing runs on the GPU, so the call needs no host copy of ids:
//
//  1. the routing (one workgroup): counts the (token, slot) pairs of every expert, an
//     exclusive scan gives each expert's run of sorted positions, and a stable
//     placement writes the pairs into their runs in pair order (ids outside
//     [0, n_expert) go to one extra run).  Deterministic: no order depends on timing.
//     For the fp16 GEMM the same launch converts x: its other workgroups turn the
//     tokens' rows into fp16, four per workgroup, while the first one routes.
//  2. the product: per expert, its columns only, on the fp16 GEMM (x gathered and
//     converted once) or the fp32 GEMM (columns read through the pair index); the
//     results go straight to their y columns.
//  3. the columns of out-of-range ids are filled with NaN.
#include "q2_0_internal.h"
#include "x_to_f16.h"

namespace q2_0 {

namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kFastRuns = 512;   // runs (experts + 1) up to which the per-wave counts fit in LDS
static_assert(kFastRuns <= 1023, "kFast run indexes and the idle value fit in 10 bits");
constexpr int kRouteKeep = 4;    // chunks whose runs stay in registers between counting and placement

// The run starts from the counts cnt[0..runs) (one wave, lane = 0..63): off[b] and, in
// place of the count, cnt[b] = the run's start; the tile list and its length.  Each lane
// takes a contiguous range of runs, then a lane scan.
__device__ __forceinline__ void scan_runs(int *cnt, int runs, int n_expert, int tile_w, int *__restrict__ off,
                                          int *__restrict__ tiles, int *__restrict__ ntiles, int lane) {
    const int L = (runs + 63) / 64, b0 = lane * L;
    int sum = 0, tsum = 0;
    for (int i = 0; i < L; ++i) {
        const int b = b0 + i;
        if (b < runs) {
            const int c = cnt[b];
            sum += c;
            if (b < n_expert) tsum += (c + tile_w - 1) / tile_w;
        }
    }
    int inc = sum, tinc = tsum;
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(inc, d), tv = __shfl_up(tinc, d);
        if (lane >= d) {
            inc += v;
            tinc += tv;
        }
    }
    int acc = inc - sum, tacc = tinc - tsum;
    for (int i = 0; i < L; ++i) {
        const int b = b0 + i;
        if (b < runs) {
            const int c = cnt[b];
            off[b] = acc;
            cnt[b] = acc;   // now the run's cursor
            if (b < n_expert)
                for (int t = 0; t * tile_w < c; ++t, ++tacc) {
                    tiles[2 * tacc] = b;
                    tiles[2 * tacc + 1] = t;
                }
            acc += c;
        }
    }
    if (lane == 63) {
        off[runs] = acc;
        *ntiles = tacc;
    }
}

// off[0..n_expert+1]: run starts (off[n_expert] .. off[n_expert+1] holds the bad ids);
// perm[pos] = pair; tiles: (expert, column tile) for every tile_w-column tile of every
// expert's run, *ntiles of them.
//  * counts: one LDS counter per run;
//  * scan: one wave, each lane over a contiguous range of runs, then a lane scan, gives
//    the run starts and the tile list;
//  * stable placement, one chunk of kRouteThreads pairs at a time: a pair goes to its
//    run's cursor + the pairs of its run in earlier waves of the chunk + those in earlier
//    lanes of its own wave.  kFast: the per-wave counts of every run sit in LDS and a
//    pair's rank in its wave is the count of earlier lanes whose run
//    index matches in every bit (one ballot per bit); otherwise (many runs) each pair
//    counts the earlier pairs of its run in the chunk one by one.
template <bool kFast>
__device__ __forceinline__ void route_pairs(const int32_t *__restrict__ ids, int n_pairs, int n_expert, int tile_w,
                                            int *__restrict__ off, int *__restrict__ perm, int *__restrict__ tiles,
                                            int *__restrict__ ntiles, int *lds) {
    const int runs = n_expert + 1;
    int *cnt = lds;                                       // runs: counts, then cursors
    int *wh = lds + runs;                                 // kFast: kRouteWaves x runs
    int *tot = wh + kRouteWaves * runs;                   // kFast: runs (a chunk's counts)
    int *chunk = lds + runs;                              // !kFast: the chunk's runs
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    auto run_of = [&](int p) {
        const int e = ids[p];
        return (e >= 0 && e < n_expert) ? e : n_expert;
    };
    for (int b = tid; b < runs; b += kRouteThreads) cnt[b] = 0;
    if (kFast)
        for (int i = tid; i < kRouteWaves * runs; i += kRouteThreads) wh[i] = 0;
    __syncthreads();
    // The first kRouteKeep chunks' runs stay in registers for the placement.
    int keep[kRouteKeep];
#pragma unroll
    for (int c = 0; c < kRouteKeep; ++c) {
        const int p = c * kRouteThreads + tid;
        keep[c] = p < n_pairs ? run_of(p) : -1;
        if (keep[c] >= 0) atomicAdd(&cnt[keep[c]], 1);
    }
    for (int p = kRouteKeep * kRouteThreads + tid; p < n_pairs; p += kRouteThreads) atomicAdd(&cnt[run_of(p)], 1);
    __syncthreads();
    if (tid < 64) scan_runs(cnt, runs, n_expert, tile_w, off, tiles, ntiles, lane);
    __syncthreads();
    for (int c0 = 0, ci = 0; c0 < n_pairs; c0 += kRouteThreads, ++ci) {
        const int p = c0 + tid;
        int b = -1;
#pragma unroll
        for (int c = 0; c < kRouteKeep; ++c) b = ci == c ? keep[c] : b;
        if (ci >= kRouteKeep) b = p < n_pairs ? run_of(p) : -1;
        if constexpr (kFast) {
            // lanes of the wave with the same run: equal in every bit of the run index
            // (b < 512; the idle value -1 reads as 1023)
            const unsigned ub = (unsigned)b & 1023u;
            uint64_t same = ~0ull;
#pragma unroll
            for (int i = 0; i < 10; ++i) {
                const uint64_t m = __ballot((ub >> i) & 1u);
                same &= ((ub >> i) & 1u) ? m : ~m;
            }
            const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(same >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)same, 0u));
            if (b >= 0) atomicAdd(&wh[wv * runs + b], 1);
            __syncthreads();
            for (int r = tid; r < runs; r += kRouteThreads) {
                int c[kRouteWaves];   // all loads first: the stores below would serialize them
#pragma unroll
                for (int v = 0; v < kRouteWaves; ++v) c[v] = wh[v * runs + r];
                int sum = 0;
#pragma unroll
                for (int v = 0; v < kRouteWaves; ++v) {
                    wh[v * runs + r] = sum;
                    sum += c[v];
                }
                tot[r] = sum;
            }
            __syncthreads();
            if (b >= 0) perm[cnt[b] + wh[wv * runs + b] + rank] = p;
            __syncthreads();
            for (int r = tid; r < runs; r += kRouteThreads) {
                cnt[r] += tot[r];
                for (int v = 0; v < kRouteWaves; ++v) wh[v * runs + r] = 0;
            }
            __syncthreads();
        } else {
            chunk[tid] = b;
            __syncthreads();
            if (b >= 0) {
                int rank = 0;
                for (int q = 0; q < tid; ++q) rank += (chunk[q] == b);
                perm[cnt[b] + rank] = p;
            }
            __syncthreads();
            if (b >= 0) atomicAdd(&cnt[b], 1);
            __syncthreads();
        }
    }
}

// The same tables for at most kRouteKeep * kRouteThreads pairs and kSmallRuns runs, in
// one pass: every pair's run stays in registers, the per-wave counts of all kRouteKeep
// chunks sit side by side in LDS (slot c * kRouteWaves + w: chunk c, wave w, i.e. pair
// order), one thread per run turns its slots into an exclusive prefix and a total, the
// scan gives the run starts, and each pair goes to its run's start + its slot's prefix +
// its rank among the earlier lanes of its wave with the same run.  Four workgroup
// barriers in all, where the chunk-by-chunk placement takes four per chunk.
constexpr int kSmallRuns = 240;   // (1 + kSlots) * runs ints of LDS stay under 64 KiB
constexpr int kSlots = kRouteKeep * kRouteWaves;
static_assert(kSmallRuns <= kFastRuns, "run indexes fit the ballot rank");

__device__ __forceinline__ void route_pairs_small(const int32_t *__restrict__ ids, int n_pairs, int n_expert,
                                                  int tile_w, int *__restrict__ off, int *__restrict__ perm,
                                                  int *__restrict__ tiles, int *__restrict__ ntiles, int *lds) {
    const int runs = n_expert + 1;
    int *cnt = lds;          // runs: totals, then run starts
    int *wh = lds + runs;    // kSlots x runs: counts, then exclusive prefixes
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int i = tid; i < kSlots * runs; i += kRouteThreads) wh[i] = 0;
    __syncthreads();
    int b[kRouteKeep], rank[kRouteKeep];
#pragma unroll
    for (int c = 0; c < kRouteKeep; ++c) {
        const int p = c * kRouteThreads + tid;
        int e = -1;
        if (p < n_pairs) {
            e = ids[p];
            e = (e >= 0 && e < n_expert) ? e : n_expert;
        }
        b[c] = e;
    }
#pragma unroll
    for (int c = 0; c < kRouteKeep; ++c) {
        // lanes of the wave with the same run: equal in every bit of the run index (the
        // idle value -1 reads as 1023)
        const unsigned ub = (unsigned)b[c] & 1023u;
        uint64_t same = ~0ull;
#pragma unroll
        for (int i = 0; i < 10; ++i) {
            const uint64_t m = __ballot((ub >> i) & 1u);
            same &= ((ub >> i) & 1u) ? m : ~m;
        }
        rank[c] = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(same >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)same, 0u));
        if (b[c] >= 0) atomicAdd(&wh[(c * kRouteWaves + wv) * runs + b[c]], 1);
    }
    __syncthreads();
    for (int r = tid; r < runs; r += kRouteThreads) {
        int sum = 0;
        for (int c = 0; c < kRouteKeep; ++c) {
            int v[kRouteWaves];   // all loads first: the stores below would serialize them
#pragma unroll
            for (int w = 0; w < kRouteWaves; ++w) v[w] = wh[(c * kRouteWaves + w) * runs + r];
#pragma unroll
            for (int w = 0; w < kRouteWaves; ++w) {
                wh[(c * kRouteWaves + w) * runs + r] = sum;
                sum += v[w];
            }
        }
        cnt[r] = sum;
    }
    __syncthreads();
    if (tid < 64) scan_runs(cnt, runs, n_expert, tile_w, off, tiles, ntiles, lane);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kRouteKeep; ++c)
        if (b[c] >= 0) perm[cnt[b[c]] + wh[(c * kRouteWaves + wv) * runs + b[c]] + rank[c]] = c * kRouteThreads + tid;
}

bool route_is_small(int n_pairs, int n_expert) {
    return n_pairs <= kRouteKeep * kRouteThreads && n_expert + 1 <= kSmallRuns;
}

size_t route_small_lds_bytes(int runs) { return (size_t)runs * (1 + kSlots) * 4; }

__global__ __launch_bounds__(kRouteThreads) void moe_route_small(const int32_t *__restrict__ ids, int n_pairs,
                                                                int n_expert, int tile_w, int *__restrict__ off,
                                                                int *__restrict__ perm, int *__restrict__ tiles,
                                                                int *__restrict__ ntiles) {
    extern __shared__ int lds[];
    route_pairs_small(ids, n_pairs, n_expert, tile_w, off, perm, tiles, ntiles, lds);
}

template <bool kFast>
__global__ __launch_bounds__(kRouteThreads) void moe_route(const int32_t *__restrict__ ids, int n_pairs,
                                                          int n_expert, int tile_w, int *__restrict__ off,
                                                          int *__restrict__ perm, int *__restrict__ tiles,
                                                          int *__restrict__ ntiles) {
    extern __shared__ int lds[];
    route_pairs<kFast>(ids, n_pairs, n_expert, tile_w, off, perm, tiles, ntiles, lds);
}

// Workgroup 0 routes (as moe_route_small or moe_route<true>); workgroup b > 0 converts x rows 4(b-1) ..
// 4(b-1)+3 for the fp16 GEMM, 256 threads each (rows past nx: the part idles).
constexpr int kConvertParts = kRouteThreads / 256;
template <bool kSmall, bool kVec, typename XT>
__global__ __launch_bounds__(kRouteThreads) void moe_route_convert(
    const int32_t *__restrict__ ids, int n_pairs, int n_expert, int tile_w, int *__restrict__ off,
    int *__restrict__ perm, int *__restrict__ tiles, int *__restrict__ ntiles, const XT *__restrict__ x,
    int64_t ldx, int K, _Float16 *__restrict__ x16, int *__restrict__ xe, XGather gather, int nx) {
    extern __shared__ int lds[];
    if (blockIdx.x == 0) {
        if (kSmall)
            route_pairs_small(ids, n_pairs, n_expert, tile_w, off, perm, tiles, ntiles, lds);
        else
            route_pairs<true>(ids, n_pairs, n_expert, tile_w, off, perm, tiles, ntiles, lds);
        return;
    }
    const int part = threadIdx.x >> 8;
    const int64_t n = (int64_t)(blockIdx.x - 1) * kConvertParts + part;
    convert_column<kVec, XT, false>(n < nx, x, ldx, K, x16, xe, gather, 0, n, threadIdx.x & 255,
                                    reinterpret_cast<float *>(lds) + 4 * part);
}

// y columns of pairs with out-of-range ids: quiet NaN.
__global__ __launch_bounds__(256) void moe_fill_bad(const int *__restrict__ off, const int *__restrict__ perm,
                                                    int n_expert, int64_t M, float *__restrict__ y, int64_t ldy) {
    const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (m >= M) return;
    for (int j = off[n_expert]; j < off[n_expert + 1]; ++j)
        y[(int64_t)perm[j] * ldy + m] = __builtin_nanf("");
}

size_t a256(size_t v) { return (v + 255) & ~(size_t)255; }
}  // namespace

// Routing tables, each 256-byte aligned: off (n_expert + 2), perm (n_pairs), ntiles (1),
// tiles (2 per possible entry).
size_t moe_route_bytes(int64_t n_expert, int64_t n_pairs, int tile_w) {
    return a256((size_t)(n_expert + 2) * 4) + a256((size_t)n_pairs * 4) + 256 +
           a256((size_t)moe_max_tiles(n_expert, n_pairs, tile_w) * 8);
}

namespace {

// The routing tables' places in ws (layout of moe_route_bytes).
struct RouteTables {
    int *off, *perm, *tiles, *ntiles;
};
RouteTables route_tables(int n_pairs, int n_expert, void *ws) {
    uint8_t *p = static_cast<uint8_t *>(ws);
    RouteTables t;
    t.off = reinterpret_cast<int *>(p);
    p += a256((size_t)(n_expert + 2) * 4);
    t.perm = reinterpret_cast<int *>(p);
    p += a256((size_t)n_pairs * 4);
    t.ntiles = reinterpret_cast<int *>(p);
    p += 256;
    t.tiles = reinterpret_cast<int *>(p);
    return t;
}

size_t route_lds_bytes(int runs) { return (size_t)runs * (2 + kRouteWaves) * 4; }

}  // namespace

bool moe_route_converts(int n_expert) { return n_expert + 1 <= kFastRuns; }

hipError_t launch_moe_route_convert(const int32_t *ids, int n_pairs, int n_expert, int n_used, int x_slots,
                                    int tile_w, void *ws, MoeRoute *r, const void *x, Act xt, int64_t ldx, int K,
                                    void *scratch, hipStream_t s) {
    if (!moe_route_converts(n_expert)) return hipErrorInvalidValue;
    const RouteTables t = route_tables(n_pairs, n_expert, ws);
    *r = MoeRoute{t.off, t.perm, t.tiles, t.ntiles, n_expert, n_pairs, n_used, x_slots, tile_w};
    uint8_t *sp = static_cast<uint8_t *>(scratch);
    _Float16 *x16 = reinterpret_cast<_Float16 *>(sp);
    int *xe = reinterpret_cast<int *>(sp + a256((size_t)n_pairs * K * 2));   // as launch_gemm_f16_moe
    const int nx = moe_x_rows(n_pairs, n_used, x_slots);
    const unsigned grid = 1u + (unsigned)((nx + kConvertParts - 1) / kConvertParts);
    const bool small = route_is_small(n_pairs, n_expert);
    const size_t lds = small ? route_small_lds_bytes(n_expert + 1) : route_lds_bytes(n_expert + 1);
    const bool vec = ((uintptr_t)x % (4 * act_bytes(xt)) == 0) && (ldx % 4 == 0);
    const XGather ident{nullptr, n_used, x_slots};
    return with_act(xt, [&](auto tag) -> hipError_t {
        using XT = decltype(tag);
        const XT *xp = static_cast<const XT *>(x);
#define Q2_0_ROUTE_CONVERT(SMALL, VEC)                                                                          \
    moe_route_convert<SMALL, VEC, XT><<<grid, kRouteThreads, lds, s>>>(ids, n_pairs, n_expert, tile_w, t.off,  \
                                                                        t.perm, t.tiles, t.ntiles, xp, ldx, K,  \
                                                                        x16, xe, ident, nx)
        if (small && vec)
            Q2_0_ROUTE_CONVERT(true, true);
        else if (small)
            Q2_0_ROUTE_CONVERT(true, false);
        else if (vec)
            Q2_0_ROUTE_CONVERT(false, true);
        else
            Q2_0_ROUTE_CONVERT(false, false);
#undef Q2_0_ROUTE_CONVERT
        return hipGetLastError();
    });
}

hipError_t launch_moe_route(const int32_t *ids, int n_pairs, int n_expert, int n_used, int x_slots, int tile_w,
                            void *ws, MoeRoute *r, hipStream_t s) {
    const RouteTables t = route_tables(n_pairs, n_expert, ws);
    *r = MoeRoute{t.off, t.perm, t.tiles, t.ntiles, n_expert, n_pairs, n_used, x_slots, tile_w};
    int *off = t.off, *perm = t.perm, *tiles = t.tiles, *ntiles = t.ntiles;
    const int runs = n_expert + 1;
    if (route_is_small(n_pairs, n_expert))
        moe_route_small<<<1, kRouteThreads, route_small_lds_bytes(runs), s>>>(ids, n_pairs, n_expert, tile_w, off,
                                                                              perm, tiles, ntiles);
    else if (runs <= kFastRuns)
        moe_route<true><<<1, kRouteThreads, route_lds_bytes(runs), s>>>(ids, n_pairs, n_expert, tile_w, off, perm,
                                                                        tiles, ntiles);
    else
        moe_route<false><<<1, kRouteThreads, (size_t)(runs + kRouteThreads) * 4, s>>>(ids, n_pairs, n_expert, tile_w,
                                                                                    off, perm, tiles, ntiles);
    return hipGetLastError();
}

hipError_t launch_moe_fill_bad(const MoeRoute &r, int64_t M, float *y, int64_t ldy, hipStream_t s) {
    moe_fill_bad<<<(unsigned)((M + 255) / 256), 256, 0, s>>>(r.off, r.perm, r.n_expert, M, y, ldy);
    return hipGetLastError();
}

}  // namespace q2_0
