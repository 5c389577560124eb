// Prefill GEMM on the gfx950 matrix cores: y[n][m] = sum_k W[m][k] x[n][k] with W in
// Q2_0, x rounded to fp16, f32 accumulation.
//
// bisque.today "WebGPU: add Q2_0 support": the tiled matrix multiply unpacks 16
// codes per thread into shared memory as half precision.  Here each thread unpacks
// one 32-bit code word (16 weights) of one row per 64-k step straight into the LDS
// tile as fp16 d*(q-1) -- exact, because d is a half and |q-1| <= 2 -- using the
// fp16-pair decode of the mat-vec (OR the code under a magic exponent, one packed
// subtract) and one packed multiply by d.
//
//  * x is converted once per call into the caller's workspace as fp16, each column
//    scaled by a power of two that keeps it inside fp16's normal range (undone on
//    the results), and within every group of 16 k its order is permuted to (0, 8,
//    1, 9, ..., 7, 15): the order in which the pair decode emits a word's 16
//    weights.  A and B then share the k order without any shuffling.
//  * Workgroup tile 128 (m) x 128 (n), four waves of 64 x 64, each a 2 x 2 grid of
//    v_mfma_f32_32x32x16_f16; one Q2_0 block (64 k) per step.
//  * LDS is double buffered (one barrier per step); the next step's code words and
//    x tile are loaded into registers two steps ahead.
//  * Tiles are ordered so that all workgroups on one XCD (dispatch is round-robin
//    over the 8 XCDs) share one 128-column slice of x, which then stays in that
//    XCD's L2.
#include "q2_0_internal.h"
#include "mat_vec_common.h"

namespace q2_0 {

namespace {

constexpr int GM = 128, GN = 128, GK = 64;
constexpr int GLD = GK + 8;   // fp16 row stride in LDS (144 B): 8 consecutive rows hit distinct banks

// x (N columns of K floats) -> fp16, k permuted inside each 16-group, one workgroup
// per column.  The column is scaled by 2^e (e = xe[n]) so that its max |x| lands in
// [2^14, 2^15): fp16 then neither overflows (|x| > 65504) nor falls into its
// subnormal range, where the relative error would exceed 2^-11.  The GEMM multiplies
// the column's results by 2^-e.
template <bool kVec>
__global__ __launch_bounds__(256) void x_to_f16_perm(const float *__restrict__ x, int64_t ldx, int K,
                                                     _Float16 *__restrict__ x16, int *__restrict__ xe) {
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int64_t n = blockIdx.x;
    const float *col = x + n * ldx;
    const int groups = K / 16;
    float m = 0.f;
    for (int gi = tid; gi < groups; gi += 256) {
        const float *src = col + 16 * gi;
        if (kVec) {
#pragma unroll
            for (int q = 0; q < 4; ++q) m = fmaxf(m, max_abs4(reinterpret_cast<const float4_t *>(src)[q]));
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) m = fmaxf(m, fabsf(src[q]));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    const int e = column_exponent(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
    if (tid == 0) xe[n] = e;
    for (int gi = tid; gi < groups; gi += 256) {
        const float *src = col + 16 * gi;
        float v[16];
        if (kVec) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4_t t = reinterpret_cast<const float4_t *>(src)[q];
                v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) v[q] = src[q];
        }
        uint32_t o[8];
#pragma unroll
        for (int s = 0; s < 8; ++s)
            o[s] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)__builtin_amdgcn_ldexpf(v[s], e),
                                                        (_Float16)__builtin_amdgcn_ldexpf(v[s + 8], e)});
        u32x4_t *dst = reinterpret_cast<u32x4_t *>(x16 + n * K + 16 * gi);
        dst[0] = u32x4_t{o[0], o[1], o[2], o[3]};
        dst[1] = u32x4_t{o[4], o[5], o[6], o[7]};
    }
}

// 16 weights of one code word as fp16 d*(q-1), in pair order (code s of the low
// half, code s of the high half), s = 0..7.
__device__ __forceinline__ void dequant_word_f16(uint32_t word, uint32_t d2, const PairMasks &pm,
                                                 uint32_t out[8]) {
    const uint32_t hi = word >> 10;
    out[0] = pair_qm1<0>(word, pm); out[1] = pair_qm1<1>(word, pm);
    out[2] = pair_qm1<2>(word, pm); out[3] = pair_qm1<3>(word, pm);
    out[4] = pair_qm1<4>(word, pm); out[5] = pair_qm1<0>(hi, pm);
    out[6] = pair_qm1<1>(hi, pm);   out[7] = pair_qm1<2>(hi, pm);
    const half2_t dd = __builtin_bit_cast(half2_t, d2);
#pragma unroll
    for (int s = 0; s < 8; ++s)
        out[s] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, out[s]) * dd);
}

struct WRegs {
    uint32_t d2[2];     // half scale in both halves
    uint32_t word[2];
};

}  // namespace

// splits > 1: workgroup (tile, split) covers blocks [split*nbs, (split+1)*nbs) and writes
// its partial sum to part + split*N*M (column n at n*M); the reduce kernel adds them.
__global__ __launch_bounds__(256, 2) void gemm_f16_mfma(const uint8_t *__restrict__ w, int M, int nb,
                                                        const _Float16 *__restrict__ x16,
                                                        const int *__restrict__ xe, int N,
                                                        float *__restrict__ y, int64_t ldy,
                                                        int tiles_m, int tiles_n, int xcd_map,
                                                        int splits, float *__restrict__ part) {
    __shared__ __attribute__((aligned(16))) _Float16 As[2][GM * GLD];
    __shared__ __attribute__((aligned(16))) _Float16 Bs[2][GN * GLD];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;   // 64 x 64 sub-tile of this wave

    // ---- tile of this workgroup.  xcd_map: XCD j = blockIdx % 8 handles column tile
    // j % tiles_n and every (8 / tiles_n)-th row tile.
    int tm, tn;
    const int split = blockIdx.x % splits;
    {
        const int b = blockIdx.x / splits;
        if (xcd_map) {
            const int j = b & 7, l = b >> 3;
            const int per = 8 / tiles_n;     // XCDs per column tile
            tn = j % tiles_n;
            tm = l * per + j / tiles_n;
        } else {
            tn = b % tiles_n;
            tm = b / tiles_n;
        }
    }
    const int m0 = tm * GM, n0 = tn * GN;
    const int K = nb * kBlockWeights;
    const int64_t rowbytes = (int64_t)nb * kBlockBytes;
    const int nbs = nb / splits;                 // blocks of this split
    const int kb0 = split * nbs;

    // ---- loader roles: two code words (rows r0, r0 + 64; word g) and four 16-byte x chunks.
    // Rows past M and columns past N read row / column 0 instead: they only feed
    // outputs that are never stored, so the loads need no guard (and no branch).
    const int g = tid & 3, r0 = tid >> 2;
    const uint8_t *wrow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = m0 + r0 + 64 * i;
        wrow[i] = w + (int64_t)(row < M ? row : 0) * rowbytes + (int64_t)kb0 * kBlockBytes;
    }
    const _Float16 *xcol[4];
    int xn[4], xpart[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = tid + 256 * q;
        xn[q] = c >> 3;
        xpart[q] = c & 7;
        const int n = n0 + xn[q];
        xcol[q] = x16 + (int64_t)(n < N ? n : 0) * K + (int64_t)kb0 * GK + 8 * xpart[q];
    }

    // Loads of a step past the last are clamped to the last block (harmless reloads),
    // so every step issues the same loads and the wait counts stay exact.
    auto load_w = [&](int blk, WRegs &r) {
        blk = min(blk, nbs - 1);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint16_t *b16 = reinterpret_cast<const uint16_t *>(wrow[i] + (int64_t)blk * kBlockBytes);
            const uint32_t d = b16[0];
            r.d2[i] = d | (d << 16);
            r.word[i] = (uint32_t)b16[1 + 2 * g] | ((uint32_t)b16[2 + 2 * g] << 16);
        }
    };
    auto load_x = [&](int blk, u32x4_t (&r)[4]) {
        blk = min(blk, nbs - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = *reinterpret_cast<const u32x4_t *>(xcol[q] + (int64_t)blk * GK);
    };
    const PairMasks pm;
    auto store_stage = [&](int buf, const WRegs &wr, const u32x4_t (&xr)[4]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint32_t o[8];
            dequant_word_f16(wr.word[i], wr.d2[i], pm, o);
            u32x4_t *dst = reinterpret_cast<u32x4_t *>(&As[buf][(r0 + 64 * i) * GLD + 16 * g]);
            dst[0] = u32x4_t{o[0], o[1], o[2], o[3]};
            dst[1] = u32x4_t{o[4], o[5], o[6], o[7]};
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<u32x4_t *>(&Bs[buf][xn[q] * GLD + 8 * xpart[q]]) = xr[q];
    };

    float16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = float16_t{};

    // A lane l: row l%32 of a 32-row sub-tile, k-slot (l/32)*8; B lane: column l%32.
    const int frow = lane & 31, fk = (lane >> 5) * 8;
    auto mma_stage = [&](int buf) {
#pragma unroll
        for (int kk = 0; kk < GK / 16; ++kk) {
            half8_t a[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = *reinterpret_cast<const half8_t *>(&As[buf][(wm * 64 + i * 32 + frow) * GLD + kk * 16 + fk]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                bv[i] = *reinterpret_cast<const half8_t *>(&Bs[buf][(wn * 64 + i * 32 + frow) * GLD + kk * 16 + fk]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], bv[jj], acc[i][jj], 0, 0, 0);
        }
    };

    // ---- pipeline: registers hold step s+1 while step s computes; loads run two steps ahead
    WRegs wA, wB;
    u32x4_t xA[4], xB[4];
    load_w(0, wA);
    load_x(0, xA);
    load_w(1, wB);
    load_x(1, xB);
    store_stage(0, wA, xA);
    load_w(2, wA);
    load_x(2, xA);
    __syncthreads();

    // Two steps per iteration so that the register sets alternate statically.  The loop
    // has no exit in the middle (an exit there makes the compiler keep the
    // accumulators in two register sets and copy between them every iteration); an
    // odd last step runs after it.
    int s = 0;
    for (; s + 1 < nbs; s += 2) {
        mma_stage(0);
        store_stage(1, wB, xB);          // step s+1
        load_w(s + 3, wB);
        load_x(s + 3, xB);
        __syncthreads();
        mma_stage(1);
        store_stage(0, wA, xA);          // step s+2 (a clamped duplicate past the end)
        load_w(s + 4, wA);
        load_x(s + 4, xA);
        __syncthreads();
    }
    if (s < nbs) mma_stage(0);

    // ---- epilogue: D lane l, register v -> row 8*(v/4) + 4*(l/32) + v%4, column l%32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int n = n0 + wn * 64 + jj * 32 + (lane & 31);
            if (n >= N) continue;
            float *yc = (splits > 1) ? part + ((int64_t)split * N + n) * M : y + (int64_t)n * ldy;
            const int ye = -xe[n];   // undo the column's staging scale
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int m = m0 + wm * 64 + i * 32 + 8 * v4 + 4 * (lane >> 5);
                float4_t val;
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = __builtin_amdgcn_ldexpf(acc[i][jj][4 * v4 + e], ye);
                if (m + 3 < M && ((((uintptr_t)(yc + m)) & 15) == 0)) {
                    *reinterpret_cast<float4_t *>(yc + m) = val;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (m + e < M) yc[m + e] = val[e];
                }
            }
        }
}

// y[n][m] = sum over splits of part[split][n][m], in split order.
__global__ __launch_bounds__(256) void gemm_split_reduce(const float *__restrict__ part, int splits, int M,
                                                         int64_t N, float *__restrict__ y, int64_t ldy) {
    const int64_t total = N * M;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t n = i / M, m = i - n * M;
        float acc = part[i];
        for (int sp = 1; sp < splits; ++sp) acc += part[(int64_t)sp * total + i];
        y[n * ldy + m] = acc;
    }
}

namespace {

// K splits for a GEMM: enough workgroups for two per CU when the tile grid alone is
// smaller, each split keeping at least 8 blocks; splits divide K/64.
int gemm_splits(int64_t M, int64_t N, int nb) {
    const int64_t tiles = ((M + GM - 1) / GM) * ((N + GN - 1) / GN);
    int sp = 1;
    while (tiles * sp < 512 && sp < 8 && nb % (2 * sp) == 0 && nb / (2 * sp) >= 8) sp *= 2;
    return sp;
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

// Workspace: fp16 x (N*K halves), the column exponents (N ints), then split-K partials.
size_t gemm_f16_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    const int sp = gemm_splits(M, N, (int)(K / kBlockWeights));
    return align256((size_t)N * K * 2) + align256((size_t)N * 4) + (sp > 1 ? align256((size_t)sp * N * M * 4) : 0);
}

hipError_t launch_gemm_f16_v2(const uint8_t *w, int64_t M, int nb, const float *x, int64_t ldx,
                              int64_t N, float *y, int64_t ldy, void *workspace, hipStream_t s) {
    const int K = nb * kBlockWeights;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    _Float16 *x16 = reinterpret_cast<_Float16 *>(ws);
    int *xe = reinterpret_cast<int *>(ws + align256((size_t)N * K * 2));
    float *part = reinterpret_cast<float *>(ws + align256((size_t)N * K * 2) + align256((size_t)N * 4));
    if (((uintptr_t)x % 16 == 0) && (ldx % 4 == 0))
        x_to_f16_perm<true><<<(unsigned)N, 256, 0, s>>>(x, ldx, K, x16, xe);
    else
        x_to_f16_perm<false><<<(unsigned)N, 256, 0, s>>>(x, ldx, K, x16, xe);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int tiles_m = (int)((M + GM - 1) / GM), tiles_n = (int)((N + GN - 1) / GN);
    const int per = (tiles_n <= 8 && 8 % tiles_n == 0) ? 8 / tiles_n : 0;
    const int splits = gemm_splits(M, N, nb);
    const int xcd_map = (splits == 1 && per != 0 && tiles_m % per == 0) ? 1 : 0;
    gemm_f16_mfma<<<tiles_m * tiles_n * splits, 256, 0, s>>>(w, (int)M, nb, x16, xe, (int)N, y, ldy, tiles_m,
                                                              tiles_n, xcd_map, splits, part);
    e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const int64_t total = N * M;
    const int rgrid = (int)((total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192);
    gemm_split_reduce<<<rgrid, 256, 0, s>>>(part, splits, (int)M, N, y, ldy);
    return hipGetLastError();
}

}  // namespace q2_0
