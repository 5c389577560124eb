// mul_mat_vec: y = W x for N = 1..8 activation columns, fp32-grade.
//
// bisque.today, "WebGPU: add Q2_0 support", the matrix-vector paragraph: there each
// block goes to four threads, one 32-bit code word (16 weights) apiece; every thread
// fetches the scale with its word, sums (q - 1) * x over its 16 codes and applies the
// scale to that partial sum a single time.
//
// Generic kernel (any row alignment, any K): one wave per output row; lane l takes
// code words l, l+64, ... of the row, forms the 16-term partial sum per column in
// f32, scales it by d and accumulates; the 64 lane sums are combined with a
// butterfly.  Summation depth per output: 16 + K/1024 + 6, far below what the
// 1e-5 relative bound allows (about 160 f32 roundings).
#include <climits>

#include "q2_0_internal.h"
#include "mat_vec_common.h"

namespace q2_0 {

template <int NC, bool kVecX, typename XT>
__global__ __launch_bounds__(256) void mat_vec_generic(const uint8_t *__restrict__ w, int64_t M,
                                                       int nb, const XT *__restrict__ x,
                                                       int64_t ldx, float *__restrict__ y,
                                                       int64_t ldy) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const uint8_t *wr = w + row * (int64_t)nb * kBlockBytes;
    const int words = nb * 4;
    float acc[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n) acc[n] = 0.f;
    for (int t = lane; t < words; t += 64) {
        const uint16_t *blk16 = reinterpret_cast<const uint16_t *>(wr + (t >> 2) * kBlockBytes);
        const float d = half_bits_to_float(blk16[0]);
        const uint32_t q = load_word_u16x2(blk16, t & 3);
        float qm1[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) qm1[i] = (float)((int)((q >> (2 * i)) & 3u) - 1);
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const XT *xp = x + n * ldx + t * 16;
            float xv[16];
            if (kVecX) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4_t v = load_act4(xp + 4 * j);
                    xv[4 * j] = v.x; xv[4 * j + 1] = v.y; xv[4 * j + 2] = v.z; xv[4 * j + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) xv[i] = act_to_f32(xp[i]);
            }
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) s = __builtin_fmaf(qm1[i], xv[i], s);
            acc[n] = __builtin_fmaf(d, s, acc[n]);
        }
    }
#pragma unroll
    for (int n = 0; n < NC; ++n) {
        float v = acc[n];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) y[n * ldy + row] = v;
    }
}

template <int NC, typename XT>
static void launch_generic_nc(const uint8_t *w, int64_t M, int nb, const XT *x, int64_t ldx,
                              float *y, int64_t ldy, hipStream_t s, bool vec) {
    dim3 grid((unsigned)((M + 3) / 4));
    if (vec)
        mat_vec_generic<NC, true, XT><<<grid, 256, 0, s>>>(w, M, nb, x, ldx, y, ldy);
    else
        mat_vec_generic<NC, false, XT><<<grid, 256, 0, s>>>(w, M, nb, x, ldx, y, ldy);
}

// Fast-path choice.  Rows 16-byte aligned and x 16-byte aligned: the MFMA kernels.
// Matrices of at least kStreamRows rows, and every group launch, stream with whole-K
// waves: one weight row per lane for N <= 2 (mat_vec_bcast.hip), 16-row tiles
// otherwise (mat_vec_stream.hip).  Smaller single matrices split K over the waves of a
// workgroup to fill the chip.  Anything else takes the generic kernel.
constexpr int64_t kStreamRows = 16384;

static int stream_tile_rows(int N) { return N <= 2 ? kMvBcastRows : kMvTile; }

// The broadcast kernel (N <= 2) stages the activation in windows, so every K fits; the
// 16-row-tile kernel (N >= 3) stages all of K where that still leaves 8 or more resident
// waves per CU (groups and batches go through it only then), and a single matrix of at
// least kStreamRows rows with a longer K runs it over chunks of whole stages.  Smaller
// matrices with such a K take the K-split kernel, faster there than chunked launches.
static bool stream_fits(int N, int nb) {
    if (N <= 2) return true;
    int resident = 0;
    const int waves = mat_vec_stream_waves(N, nb, &resident);
    return waves > 0 && resident >= 8;
}
static bool stream_fits_chunked(int N, int nb) { return stream_fits(N, nb) || mat_vec_stream_chunk_blocks(N, nb) > 0; }

// grp counts tiles of stream_tile_rows(N) rows; all its matrices share x
static hipError_t launch_streaming(const MvGroup &grp, int nb, const void *x, Act xt, int64_t ldx, int N,
                                   hipStream_t s) {
    if (N <= 2) {
        const MvSegDesc d{x, ldx, nb, 0, grp.total_tiles};
        return launch_mat_vec_bcast(grp, &d, 1, xt, N, s);
    }
    return launch_mat_vec_stream_chunked(grp, nb, x, xt, ldx, N, s);
}

hipError_t launch_mat_vec(const uint8_t *w, int64_t M, int nb, const void *x, Act xt, int64_t ldx, int N,
                          float *y, int64_t ldy, hipStream_t s) {
    if (mat_vec_mfma_eligible(w, M, nb, x, xt, ldx)) {
        if (M >= kStreamRows && stream_fits_chunked(N, nb)) {
            const int tr = stream_tile_rows(N);
            MvGroup grp;
            grp.n = 1;
            grp.p[0] = MvProblem{w, y, ldy, (int)M, 0};
            for (int i = 0; i <= kMvMaxGroup; ++i) grp.tile0[i] = i ? INT_MAX : 0;
            grp.total_tiles = (int)((M + tr - 1) / tr);
            return launch_streaming(grp, nb, x, xt, ldx, N, s);
        }
        return launch_mat_vec_mfma(w, M, nb, x, xt, ldx, N, y, ldy, s);
    }
    return launch_mat_vec_f32(w, M, nb, x, xt, ldx, N, y, ldy, s);
}

// The generic kernel: f32 arithmetic throughout, so a weight of zero contributes
// exactly nothing and the bound holds whatever the activations' range (the fp32
// precision of q2_0_mul_mat for N <= 8, and any input the fast kernels cannot take).
hipError_t launch_mat_vec_f32(const uint8_t *w, int64_t M, int nb, const void *x, Act xt, int64_t ldx, int N,
                              float *y, int64_t ldy, hipStream_t s) {
    const bool vec = ((uintptr_t)x % (4 * act_bytes(xt)) == 0) && (ldx % 4 == 0);
    return with_act(xt, [&](auto tag) -> hipError_t {
        using XT = decltype(tag);
        const XT *xp = static_cast<const XT *>(x);
        switch (N) {
            case 1: launch_generic_nc<1>(w, M, nb, xp, ldx, y, ldy, s, vec); break;
            case 2: launch_generic_nc<2>(w, M, nb, xp, ldx, y, ldy, s, vec); break;
            case 3: launch_generic_nc<3>(w, M, nb, xp, ldx, y, ldy, s, vec); break;
            case 4: launch_generic_nc<4>(w, M, nb, xp, ldx, y, ldy, s, vec); break;
            case 5: launch_generic_nc<5>(w, M, nb, xp, ldx, y, ldy, s, vec); break;
            case 6: launch_generic_nc<6>(w, M, nb, xp, ldx, y, ldy, s, vec); break;
            case 7: launch_generic_nc<7>(w, M, nb, xp, ldx, y, ldy, s, vec); break;
            case 8: launch_generic_nc<8>(w, M, nb, xp, ldx, y, ldy, s, vec); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    });
}

hipError_t launch_mat_vec_group(const q2_0_mat_vec_item *items, int64_t n_items, int nb,
                                const void *x, Act xt, int64_t ldx, int N, hipStream_t s) {
    const int tr = stream_tile_rows(N);
    int64_t i = 0;
    while (i < n_items) {
        // Gather up to kMvMaxGroup consecutive stream-eligible matrices into one launch.
        MvGroup grp;
        grp.n = 0;
        int tiles = 0;
        while (i < n_items && grp.n < kMvMaxGroup) {
            const q2_0_mat_vec_item &it = items[i];
            const uint8_t *w = static_cast<const uint8_t *>(it.w);
            if (it.M == 0) { ++i; continue; }
            const bool ok = mat_vec_mfma_eligible(w, it.M, nb, x, xt, ldx) && stream_fits(N, nb) &&
                            tiles + (it.M + tr - 1) / tr < 0x7fffffff;
            if (!ok) {
                if (grp.n) break;   // launch what is gathered first
                hipError_t e = launch_mat_vec(w, it.M, nb, x, xt, ldx, N, it.y, it.ldy, s);
                if (e != hipSuccess) return e;
                ++i;
                continue;
            }
            grp.tile0[grp.n] = tiles;
            grp.p[grp.n++] = MvProblem{w, it.y, it.ldy, (int)it.M, tiles};
            tiles += (int)((it.M + tr - 1) / tr);
            ++i;
        }
        if (grp.n) {
            for (int k = grp.n; k <= kMvMaxGroup; ++k) grp.tile0[k] = INT_MAX;
            grp.total_tiles = tiles;
            hipError_t e = launch_streaming(grp, nb, x, xt, ldx, N, s);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

// Items with their own activation and K: consecutive streaming-eligible items that share
// (x, ldx, K) form a segment; a launch takes up to kMvMaxGroup items in up to kMvMaxSegs
// segments (N <= 2) or one segment (N >= 3, whose kernel stages one activation).  Other
// items run alone.
hipError_t launch_mat_vec_batch(const q2_0_mat_vec_batch_item *items, int64_t n_items, Act xt, int N,
                                hipStream_t s) {
    const int tr = stream_tile_rows(N);
    int64_t i = 0;
    while (i < n_items) {
        MvGroup grp;
        grp.n = 0;
        int tiles = 0;
        MvSegDesc segs[kMvMaxSegs];
        int nsegs = 0;
        while (i < n_items && grp.n < kMvMaxGroup) {
            const q2_0_mat_vec_batch_item &it = items[i];
            if (it.M == 0) { ++i; continue; }
            const uint8_t *w = static_cast<const uint8_t *>(it.w);
            const int nb = (int)(it.K / kBlockWeights);
            const bool ok = mat_vec_mfma_eligible(w, it.M, nb, it.x, xt, it.ldx) && stream_fits(N, nb) &&
                            tiles + (it.M + tr - 1) / tr < 0x7fffffff;
            if (!ok) {
                if (grp.n) break;   // launch what is gathered first
                hipError_t e = launch_mat_vec(w, it.M, nb, it.x, xt, it.ldx, N, it.y, it.ldy, s);
                if (e != hipSuccess) return e;
                ++i;
                continue;
            }
            const bool same = nsegs > 0 && segs[nsegs - 1].x == it.x && segs[nsegs - 1].ldx == it.ldx &&
                              segs[nsegs - 1].nb == nb;
            if (!same) {
                if (nsegs == kMvMaxSegs || (N > 2 && nsegs == 1)) break;
                segs[nsegs++] = MvSegDesc{it.x, it.ldx, nb, tiles, tiles};
            }
            grp.tile0[grp.n] = tiles;
            grp.p[grp.n++] = MvProblem{w, it.y, it.ldy, (int)it.M, tiles};
            tiles += (int)((it.M + tr - 1) / tr);
            segs[nsegs - 1].tile1 = tiles;
            ++i;
        }
        if (grp.n) {
            for (int k = grp.n; k <= kMvMaxGroup; ++k) grp.tile0[k] = INT_MAX;
            grp.total_tiles = tiles;
            const hipError_t e = N <= 2 ? launch_mat_vec_bcast(grp, segs, nsegs, xt, N, s)
                                        : launch_mat_vec_stream_chunked(grp, segs[0].nb, segs[0].x, xt, segs[0].ldx, N, s);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace q2_0
