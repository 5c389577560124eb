// mul_mat fp32 fallback: batched Q2_0 x F32 GEMM, y[n][m] = sum_k W[m][k] x[n][k],
// fp32-grade (the fp16-MFMA GEMM is gemm_f16.hip).
//
// bisque.today, "WebGPU: add Q2_0 support", the paragraph on its three shaders: its
// tiled GEMM expands sixteen codes per thread into workgroup memory; here four
// threads per row each unpack one
// 32-bit word of the row's block into an LDS tile.
//
//  * gemm_f32: the accuracy fallback.  W is kept as f32 (q-1) with the block scale
//    apart; each block's 64-term sum is formed in f32 and multiplied by d once (as
//    the mat-vec paragraph describes), and block partials are accumulated in fp64,
//    so the only f32 roundings are the 64-deep in-block chain.
//
// Tiles: 64 rows (m) x 64 columns (n) per 256-thread workgroup, one Q2_0 block
// (64 k) per step.  Ragged M and N are handled with zero fill and masked stores.
#include "q2_0_internal.h"

namespace q2_0 {

namespace {

constexpr int BM = 64, BN = 64, BK = 64;

}  // namespace

constexpr int LDF = BM + 4;   // f32 k-major row stride (16-byte multiple)

// Expert routing: blockIdx.y indexes the routing's (expert, column tile) list; the
// workgroup's columns are that tile of the expert's run of sorted pairs, read from x
// and written to y through the pair index.
struct MoeCols {
    const int *off;       // nullptr: plain product
    const int *perm;
    const int *tiles;
    const int *ntiles;
    int n_used, x_slots;
    int64_t expert_bytes;
};

template <typename XT>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const uint8_t *__restrict__ w, int64_t M,
                                                       int nb, const XT *__restrict__ x,
                                                       int64_t ldx, int64_t N,
                                                       float *__restrict__ y, int64_t ldy, MoeCols moe) {
    __shared__ __attribute__((aligned(16))) float Wt[BK][LDF];   // (q-1), k-major
    __shared__ __attribute__((aligned(16))) float Xt[BK][LDF];   // x, k-major
    __shared__ float Ds[BM];
    const int tid = threadIdx.x;
    const int64_t m0 = (int64_t)blockIdx.x * BM;
    int64_t n0 = (int64_t)blockIdx.y * BN;
    const int r = tid >> 2, wi = tid & 3;
    const int tx = tid & 15, ty = tid >> 4;    // outputs: rows ty*4+i, columns tx*4+j

    int col0 = 0;
    if (moe.off) {
        const int t = blockIdx.y;
        if (t >= *moe.ntiles) return;   // the whole workgroup: no tile here
        const int e = moe.tiles[2 * t];
        n0 = (int64_t)moe.tiles[2 * t + 1] * BN;
        col0 = moe.off[e];
        N = moe.off[e + 1] - col0;
        w += e * moe.expert_bytes;
    }
    // x column and y column of local column n
    auto xcol_of = [&](int64_t n) -> int64_t {
        if (!moe.off) return n;
        const int p = moe.perm[col0 + n];
        return moe.x_slots == 1 ? p / moe.n_used : p;
    };
    const int64_t lm = m0 + r, ln = n0 + r;
    const uint8_t *wrow = w + (lm < M ? lm : 0) * (int64_t)nb * kBlockBytes;
    const XT *xcol = x + xcol_of(ln < N ? ln : 0) * ldx;

    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;

    for (int b = 0; b < nb; ++b) {
        if (lm < M) {
            const uint16_t *blk16 = reinterpret_cast<const uint16_t *>(wrow + b * kBlockBytes);
            const uint32_t q = load_word_u16x2(blk16, wi);
#pragma unroll
            for (int i = 0; i < 16; ++i) Wt[16 * wi + i][r] = (float)((int)((q >> (2 * i)) & 3u) - 1);
            if (wi == 0) Ds[r] = half_bits_to_float(blk16[0]);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) Wt[16 * wi + i][r] = 0.f;
            if (wi == 0) Ds[r] = 0.f;
        }
        if (ln < N) {
            const XT *xp = xcol + (int64_t)b * BK + 16 * wi;
#pragma unroll
            for (int i = 0; i < 16; ++i) Xt[16 * wi + i][r] = act_to_f32(xp[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) Xt[16 * wi + i][r] = 0.f;
        }
        __syncthreads();
        float s[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) s[i][j] = 0.f;
#pragma unroll 8
        for (int k = 0; k < BK; ++k) {
            const float4_t a = *reinterpret_cast<const float4_t *>(&Wt[k][ty * 4]);
            const float4_t bv = *reinterpret_cast<const float4_t *>(&Xt[k][tx * 4]);
            const float av[4] = {a.x, a.y, a.z, a.w};
            const float bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) s[i][j] = __builtin_fmaf(av[i], bw[j], s[i][j]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double d = (double)Ds[ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fma(d, (double)s[i][j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + tx * 4 + j;
        if (n >= N) continue;
        float *yc = y + (moe.off ? (int64_t)moe.perm[col0 + n] : n) * ldy;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = m0 + ty * 4 + i;
            if (m < M) yc[m] = (float)acc[i][j];
        }
    }
}

hipError_t launch_gemm_f32(const uint8_t *w, int64_t M, int nb, const void *x, Act xt, int64_t ldx,
                           int64_t N, float *y, int64_t ldy, hipStream_t s) {
    dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((N + BN - 1) / BN));
    return with_act(xt, [&](auto tag) -> hipError_t {
        using XT = decltype(tag);
        gemm_f32_kernel<XT><<<grid, 256, 0, s>>>(w, M, nb, static_cast<const XT *>(x), ldx, N, y, ldy,
                                                 MoeCols{nullptr, nullptr, nullptr, nullptr, 1, 1, 0});
        return hipGetLastError();
    });
}

hipError_t launch_gemm_f32_moe(const uint8_t *w, int64_t M, int nb, const void *x, Act xt, int64_t ldx,
                               const MoeRoute &r, float *y, int64_t ldy, hipStream_t s) {
    // one workgroup row per entry the tile list can have (at most 65535, which the entry
    // point checks); the entries past its length exit at once
    dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)moe_max_tiles(r.n_expert, r.n_pairs, BN));
    const MoeCols moe{r.off, r.perm, r.tiles, r.ntiles, r.n_used, r.x_slots, M * (int64_t)nb * kBlockBytes};
    return with_act(xt, [&](auto tag) -> hipError_t {
        using XT = decltype(tag);
        gemm_f32_kernel<XT><<<grid, 256, 0, s>>>(w, M, nb, static_cast<const XT *>(x), ldx, r.n_pairs, y, ldy,
                                                 moe);
        return hipGetLastError();
    });
}

}  // namespace q2_0
