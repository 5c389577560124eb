// mul_mat: batched Q2_0 x F32 GEMM (prefill), y[n][m] = sum_k W[m][k] x[n][k].
//
// bisque.today, "WebGPU: add Q2_0 support": the tiled matrix multiply unpacks 16
// codes per thread into shared memory as half precision.  Here the same split of
// a block over four threads (one 32-bit word each) fills an LDS tile; on gfx950
// the tile feeds the matrix cores.
//
//  * gemm_f16: the W tile is stored in LDS as fp16 d*(q-1) -- exact, because d is a
//    half and |q-1| <= 2 -- and the x tile as fp16 (nearest-even).  MFMA
//    v_mfma_f32_32x32x16_f16 accumulates in f32.  Error: x rounding (2^-12 relative)
//    plus f32 accumulation, well inside 2e-3 of sum|W x|.
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
constexpr int LDH = BK + 8;   // fp16 row stride (144 B) breaks the 128 B bank period

// Dequantize 16 codes of word q with scale d to fp16 d*(q-1) (exact).
__device__ __forceinline__ void dequant16_f16(uint32_t q, float d, _Float16 *dst) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
        dst[i] = (_Float16)((float)((int)((q >> (2 * i)) & 3u) - 1) * d);
}

}  // namespace

__global__ __launch_bounds__(256) void gemm_f16_kernel(const uint8_t *__restrict__ w, int64_t M,
                                                       int nb, const float *__restrict__ x,
                                                       int64_t ldx, int64_t N,
                                                       float *__restrict__ y, int64_t ldy) {
    __shared__ __attribute__((aligned(16))) _Float16 As[BM][LDH];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[BN][LDH];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t m0 = (int64_t)blockIdx.x * BM;
    const int64_t n0 = (int64_t)blockIdx.y * BN;
    const int r = tid >> 2, wi = tid & 3;     // loader: row/col r, word / k-chunk wi
    const int wm = wave & 1, wn = wave >> 1;  // 32x32 sub-tile of this wave

    const int64_t lm = m0 + r, ln = n0 + r;
    const uint8_t *wrow = w + (lm < M ? lm : 0) * (int64_t)nb * kBlockBytes;
    const float *xcol = x + (ln < N ? ln : 0) * ldx;

    float16_t acc = {};
    for (int b = 0; b < nb; ++b) {
        // ---- stage W block b of 64 rows and x[k0:k0+64] of 64 columns as fp16
        {
            _Float16 hv[16];
            if (lm < M) {
                const uint16_t *blk16 = reinterpret_cast<const uint16_t *>(wrow + b * kBlockBytes);
                dequant16_f16(load_word_u16x2(blk16, wi), half_bits_to_float(blk16[0]), hv);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) hv[i] = (_Float16)0.f;
            }
            half8_t *dst = reinterpret_cast<half8_t *>(&As[r][16 * wi]);
            dst[0] = half8_t{hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]};
            dst[1] = half8_t{hv[8], hv[9], hv[10], hv[11], hv[12], hv[13], hv[14], hv[15]};
        }
        {
            _Float16 hv[16];
            if (ln < N) {
                const float *xp = xcol + (int64_t)b * BK + 16 * wi;
#pragma unroll
                for (int i = 0; i < 16; ++i) hv[i] = (_Float16)xp[i];
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) hv[i] = (_Float16)0.f;
            }
            half8_t *dst = reinterpret_cast<half8_t *>(&Bs[r][16 * wi]);
            dst[0] = half8_t{hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]};
            dst[1] = half8_t{hv[8], hv[9], hv[10], hv[11], hv[12], hv[13], hv[14], hv[15]};
        }
        __syncthreads();
        // ---- 4 MFMAs of 16 k each; lane l supplies row/col l%32, k-group l/32 (8 k)
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const half8_t a = *reinterpret_cast<const half8_t *>(&As[wm * 32 + (lane & 31)][kk * 16 + (lane >> 5) * 8]);
            const half8_t bv = *reinterpret_cast<const half8_t *>(&Bs[wn * 32 + (lane & 31)][kk * 16 + (lane >> 5) * 8]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bv, acc, 0, 0, 0);
        }
        __syncthreads();
    }
    // ---- D layout of the 32x32 MFMA: lane l, register v -> row 8*(v/4) + 4*(l/32) + v%4,
    //      column l%32.
    const int64_t n = n0 + wn * 32 + (lane & 31);
    if (n < N) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t m = m0 + wm * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
            if (m < M) y[n * ldy + m] = acc[v];
        }
    }
}

constexpr int LDF = BM + 4;   // f32 k-major row stride (16-byte multiple)

__global__ __launch_bounds__(256) void gemm_f32_kernel(const uint8_t *__restrict__ w, int64_t M,
                                                       int nb, const float *__restrict__ x,
                                                       int64_t ldx, int64_t N,
                                                       float *__restrict__ y, int64_t ldy) {
    __shared__ __attribute__((aligned(16))) float Wt[BK][LDF];   // (q-1), k-major
    __shared__ __attribute__((aligned(16))) float Xt[BK][LDF];   // x, k-major
    __shared__ float Ds[BM];
    const int tid = threadIdx.x;
    const int64_t m0 = (int64_t)blockIdx.x * BM;
    const int64_t n0 = (int64_t)blockIdx.y * BN;
    const int r = tid >> 2, wi = tid & 3;
    const int tx = tid & 15, ty = tid >> 4;    // outputs: rows ty*4+i, columns tx*4+j

    const int64_t lm = m0 + r, ln = n0 + r;
    const uint8_t *wrow = w + (lm < M ? lm : 0) * (int64_t)nb * kBlockBytes;
    const float *xcol = x + (ln < N ? ln : 0) * ldx;

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
            const float *xp = xcol + (int64_t)b * BK + 16 * wi;
#pragma unroll
            for (int i = 0; i < 16; ++i) Xt[16 * wi + i][r] = xp[i];
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
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t m = m0 + ty * 4 + i;
            if (m < M) y[n * ldy + m] = (float)acc[i][j];
        }
    }
}

hipError_t launch_gemm_f16(const uint8_t *w, int64_t M, int nb, const float *x, int64_t ldx,
                           int64_t N, float *y, int64_t ldy, hipStream_t s) {
    dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((N + BN - 1) / BN));
    gemm_f16_kernel<<<grid, 256, 0, s>>>(w, M, nb, x, ldx, N, y, ldy);
    return hipGetLastError();
}

hipError_t launch_gemm_f32(const uint8_t *w, int64_t M, int nb, const float *x, int64_t ldx,
                           int64_t N, float *y, int64_t ldy, hipStream_t s) {
    dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((N + BN - 1) / BN));
    gemm_f32_kernel<<<grid, 256, 0, s>>>(w, M, nb, x, ldx, N, y, ldy);
    return hipGetLastError();
}

}  // namespace q2_0
