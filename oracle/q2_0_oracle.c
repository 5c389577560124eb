/*
 * Q2_0 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 implementation of what the Q2_0 hot path computes.  Only
 * the tests, the package smoke check and the benchmark's CPU-baseline leg load
 * it; the product library never does, and the two share no code.
 *
 * Sources (the pages this follows):
 *  [P1] bisque.today, "WebGPU: add Q2_0 support" (llama.cpp PR 30914):
 *       the paragraph on the block format (64 weights in 18 bytes, a half
 *       precision scale d first, then four 32-bit words of sixteen 2-bit codes,
 *       code q decodes to (q - 1) * d) and the paragraph on the mat-vec kernel
 *       (the codes of a word are taken two bits apiece, lowest first; the scale is applied
 *       once per block, after the sum of (q - 1) * x).
 *  [P3] aisvetem.cz, "Llama.cpp umi dvoubitovy Q2_0 i na kartach NVIDIA",
 *       section "Osmnact bajtu na ctyriasedesat vah" (18 bytes / 64 weights /
 *       2.25 bpw; codes 0..3 minus one, times the scale, so -d, 0, d, 2d; the
 *       fourth level is reserved) and section "Na bezny model to neni" (the
 *       reference quantizer: the block's largest |w| is the scale, each weight
 *       goes to the nearest of the four levels).
 *
 * Readings where the pages are silent (each one is also listed in the design doc):
 *  - d and the code words are little-endian; code i of word w is weight 16w+i.
 *  - Half precision is full IEEE binary16: subnormals, +-0, +-inf and NaN.
 *  - get_rows writes the f32 value of (q - 1) * d; since d is a half and
 *    |q - 1| <= 2 the fp64 product is exact and fits f32, so the cast is exact
 *    and the sign of zero is the IEEE product's.
 *  - An out-of-range row id fills its output row with quiet NaN.
 *  - Quantizer: the scale is the half nearest (ties to even) to max |w|; codes
 *    are chosen against that rounded scale; a tie goes to the level nearer zero;
 *    a block whose rounded scale is 0 gets code 1 everywhere.
 *  - The older group-128 packing ([P3], section "Sest procent, o ktera se vedl
 *    spor": 34 bytes per 128 weights) is the group-64 block extended: a half scale,
 *    then eight little-endian words, code i of word w for weight 16w+i.
 *
 * Every function is a direct loop over the definition; parallelism is only
 * across independent output rows (OpenMP), never inside a sum.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define O_BLOCK_WEIGHTS 64
#define O_BLOCK_BYTES 18

/* IEEE binary16 -> double, from the definition: 1 sign bit, 5 exponent bits
 * with bias 15, 10 fraction bits; exponent 0 is zero/subnormal (f * 2^-24),
 * exponent 31 is inf (f == 0) or NaN. */
double oracle_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp(1024.0 + (double)f, e - 25);
    return sign ? -v : v;
}

/* double -> IEEE binary16 bits, round to nearest, ties to even; overflow to inf.
 * Works on the exact value: the candidate halves around |x| are compared by
 * their distance in fp64, which is exact for every double in half range. */
uint16_t oracle_double_to_half(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) return 0x7e00;
    if (a == 0.0) return sign;
    /* largest finite half 65504; halfway to the next (65536) is 65520 */
    if (a >= 65520.0) return sign | 0x7c00;
    /* find the two consecutive half bit patterns (non-negative) bracketing a */
    uint16_t lo = 0, hi = 0x7bff;
    while (hi - lo > 1) { /* binary search: halves are monotone in their bits */
        uint16_t mid = (uint16_t)((lo + hi) / 2);
        if (oracle_half_to_double(mid) <= a) lo = mid; else hi = mid;
    }
    if (oracle_half_to_double(hi) <= a) lo = hi; /* a at or above the top pattern */
    double vlo = oracle_half_to_double(lo);
    if (vlo == a || lo == 0x7bff) return sign | lo;
    uint16_t up = (uint16_t)(lo + 1);
    double vup = oracle_half_to_double(up);
    double dlo = a - vlo, dup = vup - a;
    uint16_t r;
    if (dlo < dup) r = lo;
    else if (dup < dlo) r = up;
    else r = (lo & 1) ? up : lo; /* tie: even fraction */
    return sign | r;
}

/* The code of weight j (0..63) of the block at b: weight j is code j%16 of
 * word j/16; on the little-endian word that is byte 2 + 4*(j/16) + (j%16)/4 of
 * the block, bits 2*(j%4)..2*(j%4)+1.  Read byte by byte on purpose. */
static int o_code(const uint8_t *b, int j) {
    int w = j / 16, i = j % 16;
    return (b[2 + 4 * w + i / 4] >> (2 * (i % 4))) & 3;
}

static double o_scale(const uint8_t *b) {
    return oracle_half_to_double((uint16_t)(b[0] | (b[1] << 8)));
}

static const uint8_t *o_block(const uint8_t *w, int64_t K, int64_t m, int64_t blk) {
    return w + (m * (K / O_BLOCK_WEIGHTS) + blk) * O_BLOCK_BYTES;
}

/* Dequantize row m into out[0..K): (q - 1) * d in fp64. */
void oracle_dequant_row(const uint8_t *w, int64_t K, int64_t m, double *out) {
    int64_t nb = K / O_BLOCK_WEIGHTS;
    for (int64_t blk = 0; blk < nb; ++blk) {
        const uint8_t *b = o_block(w, K, m, blk);
        double d = o_scale(b);
        for (int j = 0; j < O_BLOCK_WEIGHTS; ++j)
            out[blk * O_BLOCK_WEIGHTS + j] = (double)(o_code(b, j) - 1) * d;
    }
}

/* get_rows: out row r (stride ld_out floats) = row ids[r] of W, dequantized. */
void oracle_get_rows(const uint8_t *w, int64_t M, int64_t K, const int32_t *ids, int64_t n_ids,
                     float *out, int64_t ld_out) {
    int64_t nb = K / O_BLOCK_WEIGHTS;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_ids; ++r) {
        float *o = out + r * ld_out;
        int64_t m = ids[r];
        if (m < 0 || m >= M) {
            for (int64_t k = 0; k < K; ++k) o[k] = (float)NAN;
            continue;
        }
        for (int64_t blk = 0; blk < nb; ++blk) {
            const uint8_t *b = o_block(w, K, m, blk);
            double d = o_scale(b);
            for (int j = 0; j < O_BLOCK_WEIGHTS; ++j)
                o[blk * O_BLOCK_WEIGHTS + j] = (float)((double)(o_code(b, j) - 1) * d);
        }
    }
}

/* Products over a subset of rows.
 *   y[n*ldy + m]  = sum_b d_{m,b} * sum_{i<64} (q_{m,b,i} - 1) * x[n*ldx + 64b + i]
 *   bound[n*ldy+m]= sum_b |d_{m,b}| * sum_{i<64} |q - 1| * |x|
 * both in fp64, sums in index order.  rows == NULL means all M rows. */
void oracle_mul_mat_rows(const uint8_t *w, int64_t M, int64_t K, const float *x, int64_t ldx,
                         int64_t N, const int64_t *rows, int64_t n_rows, double *y, double *bound,
                         int64_t ldy) {
    int64_t nb = K / O_BLOCK_WEIGHTS;
    int64_t count = rows ? n_rows : M;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < count; ++t) {
        int64_t m = rows ? rows[t] : t;
        int64_t out_col = rows ? t : m;
        for (int64_t n = 0; n < N; ++n) {
            const float *xc = x + n * ldx;
            double acc = 0.0, accb = 0.0;
            for (int64_t blk = 0; blk < nb; ++blk) {
                const uint8_t *b = o_block(w, K, m, blk);
                double d = o_scale(b);
                double s = 0.0, sb = 0.0;
                for (int j = 0; j < O_BLOCK_WEIGHTS; ++j) {
                    double q1 = (double)(o_code(b, j) - 1);
                    double xv = (double)xc[blk * O_BLOCK_WEIGHTS + j];
                    s += q1 * xv;
                    sb += fabs(q1) * fabs(xv);
                }
                acc += d * s;
                accb += fabs(d) * sb;
            }
            y[n * ldy + out_col] = acc;
            if (bound) bound[n * ldy + out_col] = accb;
        }
    }
}

void oracle_mul_mat(const uint8_t *w, int64_t M, int64_t K, const float *x, int64_t ldx, int64_t N,
                    double *y, double *bound, int64_t ldy) {
    oracle_mul_mat_rows(w, M, K, x, ldx, N, 0, 0, y, bound, ldy);
}

/* Reference quantizer: f32 weights (M rows of K) -> packed Q2_0. */
void oracle_quantize_ref(const float *src, int64_t M, int64_t K, uint8_t *dst) {
    int64_t nb = K / O_BLOCK_WEIGHTS;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t blk = 0; blk < nb; ++blk) {
            const float *v = src + m * K + blk * O_BLOCK_WEIGHTS;
            uint8_t *b = dst + (m * nb + blk) * O_BLOCK_BYTES;
            double amax = 0.0;
            for (int j = 0; j < O_BLOCK_WEIGHTS; ++j)
                if (fabs((double)v[j]) > amax) amax = fabs((double)v[j]);
            uint16_t hb = oracle_double_to_half(amax);
            double d = oracle_half_to_double(hb);
            b[0] = (uint8_t)(hb & 0xff);
            b[1] = (uint8_t)(hb >> 8);
            memset(b + 2, 0, 16);
            for (int j = 0; j < O_BLOCK_WEIGHTS; ++j) {
                int best = 1;
                if (d != 0.0) {
                    double bestdist = INFINITY;
                    /* candidates in order of |q - 1|, so a strict '<' keeps the
                     * level nearer zero on a tie */
                    static const int order[4] = {1, 0, 2, 3};
                    for (int c = 0; c < 4; ++c) {
                        int q = order[c];
                        double dist = fabs((double)v[j] - (double)(q - 1) * d);
                        if (dist < bestdist) { bestdist = dist; best = q; }
                    }
                }
                int wd = j / 16, i = j % 16;
                b[2 + 4 * wd + i / 4] |= (uint8_t)(best << (2 * (i % 4)));
            }
        }
    }
}

/* Legacy group-128 packing: dequantize row m (K/128 blocks of 34 bytes) into
 * out[0..K) as (q - 1) * d in fp64.  Weight j of a block is code j%16 of word j/16:
 * byte 2 + 4*(j/16) + (j%16)/4, bits 2*(j%4)..2*(j%4)+1. */
void oracle_dequant_g128_row(const uint8_t *w128, int64_t K, int64_t m, double *out) {
    int64_t nb = K / 128;
    for (int64_t blk = 0; blk < nb; ++blk) {
        const uint8_t *b = w128 + (m * nb + blk) * 34;
        double d = oracle_half_to_double((uint16_t)(b[0] | (b[1] << 8)));
        for (int j = 0; j < 128; ++j) {
            int w = j / 16, i = j % 16;
            int q = (b[2 + 4 * w + i / 4] >> (2 * (i % 4))) & 3;
            out[blk * 128 + j] = (double)(q - 1) * d;
        }
    }
}

/* Legacy group-128 -> group 64: block j of a row becomes blocks 2j and 2j+1, each
 * with the legacy scale bytes, holding the code bytes of weights 0..63 and
 * 64..127 (bytes 2..17 and 18..33 of the legacy block). */
void oracle_repack_g128(const uint8_t *w128, int64_t M, int64_t K, uint8_t *dst) {
    int64_t nb = K / 128;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t blk = 0; blk < nb; ++blk) {
            const uint8_t *b = w128 + (m * nb + blk) * 34;
            for (int h = 0; h < 2; ++h) {
                uint8_t *o = dst + ((m * nb + blk) * 2 + h) * O_BLOCK_BYTES;
                o[0] = b[0];
                o[1] = b[1];
                memcpy(o + 2, b + 2 + 16 * h, 16);
            }
        }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
