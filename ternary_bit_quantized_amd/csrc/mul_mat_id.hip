// Expert ("mixture of experts") product: y[t][u] = W_{ids[t][u]} x[t][u mod x_slots].
//
// bisque.today "WebGPU: add Q2_0 support" leaves the expert mat-mul out for Q2_0 (the
// paragraph on what the change does not cover); this is that product on the same
// block decode.  The routing runs on the GPU, so the call needs no host copy of ids:
//
//  1. moe_route (one workgroup): counts the (token, slot) pairs of every expert, an
//     exclusive scan gives each expert's run of sorted positions, and a stable
//     placement writes the pairs into their runs in pair order (ids outside
//     [0, n_expert) go to one extra run).  Deterministic: no order depends on timing.
//  2. the product: per expert, its columns only, on the fp16 GEMM (x gathered and
//     converted once) or the fp32 GEMM (columns read through the pair index); the
//     results go straight to their y columns.
//  3. the columns of out-of-range ids are filled with NaN.
#include "q2_0_internal.h"

namespace q2_0 {

namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kFastRuns = 512;   // runs (experts + 1) up to which the per-wave counts fit in LDS
static_assert(kFastRuns <= 1023, "kFast run indexes and the idle value fit in 10 bits");
constexpr int kRouteKeep = 4;    // chunks whose runs stay in registers between counting and placement

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
__global__ __launch_bounds__(kRouteThreads) void moe_route(const int32_t *__restrict__ ids, int n_pairs,
                                                          int n_expert, int tile_w, int *__restrict__ off,
                                                          int *__restrict__ perm, int *__restrict__ tiles,
                                                          int *__restrict__ ntiles) {
    extern __shared__ int lds[];
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
    if (tid < 64) {
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

hipError_t launch_moe_route(const int32_t *ids, int n_pairs, int n_expert, int n_used, int x_slots, int tile_w,
                            void *ws, MoeRoute *r, hipStream_t s) {
    uint8_t *p = static_cast<uint8_t *>(ws);
    int *off = reinterpret_cast<int *>(p);
    p += a256((size_t)(n_expert + 2) * 4);
    int *perm = reinterpret_cast<int *>(p);
    p += a256((size_t)n_pairs * 4);
    int *ntiles = reinterpret_cast<int *>(p);
    p += 256;
    int *tiles = reinterpret_cast<int *>(p);
    *r = MoeRoute{off, perm, tiles, ntiles, n_expert, n_pairs, n_used, x_slots, tile_w};
    const int runs = n_expert + 1;
    if (runs <= kFastRuns)
        moe_route<true><<<1, kRouteThreads, (size_t)runs * (2 + kRouteWaves) * 4, s>>>(ids, n_pairs, n_expert, tile_w,
                                                                                    off, perm, tiles, ntiles);
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
