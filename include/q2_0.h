/*
 * q2_0.h -- C ABI of the MI355X (gfx950) Q2_0 x F32 library (libq2_0.so).
 *
 * Q2_0 storage (bisque.today, "WebGPU: add Q2_0 support" (llama.cpp PR 30914),
 * the paragraph on the block format; aisvetem.cz, "Llama.cpp umi dvoubitovy Q2_0
 * i na kartach NVIDIA", section "Osmnact bajtu na ctyriasedesat vah"):
 *   - a block is 18 bytes holding 64 weights (2.25 bits per weight);
 *   - bytes 0-1: the scale d, IEEE half precision, little-endian;
 *   - bytes 2-17: four little-endian 32-bit words; code i of word w is bits
 *     2i..2i+1 and belongs to weight 16w+i;
 *   - code q stands for the weight (q - 1) * d, i.e. -d, 0, d, 2d (code 3 is reserved by
 *     the model card but decodes to 2d and is accepted).
 *
 * Matrix layout used by every entry point:
 *   w : M rows, each K/64 consecutive blocks; row m starts at byte m*(K/64)*18.
 *   x : N activation columns of K contiguous floats; column n starts at x + n*ldx.
 *   y : N output columns of M contiguous floats;     column n starts at y + n*ldy.
 * so y[n][m] = sum_k W[m][k] * x[n][k]  (W times each activation column).
 *
 * Conventions shared by all calls:
 *   - Every pointer is a DEVICE pointer owned by the caller.  The library never
 *     allocates device memory on a call and keeps no reference after the call
 *     returns.  Its only global state is a thread-local copy of the last HIP error
 *     and a per-device flag, set once with an atomic store, that records that the
 *     kernels' shared-memory limit was raised.  Calls may come from any thread.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *     work; the caller keeps buffers alive until the stream has passed them.
 *   - Arguments are validated on the host before anything is launched; on any
 *     error nothing is written and nothing is launched.  Check order: SHAPE,
 *     then the empty no-op (M, N or n_ids == 0 returns Q2_0_OK), then NULL,
 *     LAYOUT, ALIGN, UNSUPPORTED, WORKSPACE.
 *   - No call prints, throws across the ABI or aborts.
 */
#ifndef Q2_0_H
#define Q2_0_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q2_0_BLOCK_WEIGHTS 64
#define Q2_0_BLOCK_BYTES 18

typedef enum {
    Q2_0_OK = 0,
    Q2_0_ERR_NULL = 1,        /* a required pointer is NULL */
    Q2_0_ERR_SHAPE = 2,       /* K <= 0, K % 64 != 0, a negative size, or a size beyond the limits */
    Q2_0_ERR_LAYOUT = 3,      /* ldx < K, ldy < M or ld_out < K */
    Q2_0_ERR_ALIGN = 4,       /* w not 2-byte aligned, or x / y / out / ids not aligned to their element size */
    Q2_0_ERR_UNSUPPORTED = 5, /* N > 8 for the mat-vec, or an unknown precision or activation type */
    Q2_0_ERR_WORKSPACE = 6,   /* workspace smaller than q2_0_mul_mat_workspace_bytes(), or not 16-byte aligned */
    Q2_0_ERR_HIP = 7,         /* a HIP launch failed; see q2_0_last_hip_error() */
    Q2_0_ERR_TOO_LARGE = 8    /* q2_0_mul_mat_noalloc: the call needs more than Q2_0_NOALLOC_SCRATCH_BYTES */
} q2_0_status;

typedef enum {
    Q2_0_PREC_F16_MFMA = 0,   /* fast: W as fp16 d*(q-1) (exact), x rounded to fp16, MFMA, f32 accumulate */
    Q2_0_PREC_F32 = 1,        /* accuracy fallback: W as f32 (q-1) and d, x in f32, f32 FMA, no range condition */
    Q2_0_PREC_F32_MFMA = 2    /* fp32-grade on the matrix cores: x as an fp16 hi/lo pair, per-block f32 sums
                                 added in fp64; the 1e-5 bound under the mat-vec's range condition */
} q2_0_precision;

/* Largest activation-column count of q2_0_mul_mat_vec. */
#define Q2_0_MAT_VEC_MAX_N 8

/*
 * Activation element types of the *_act entry points.  The WebGPU backend of
 * bisque.today "WebGPU: add Q2_0 support" accepts only F32 activations (the
 * paragraph on what the change leaves out); these calls add half- and
 * bfloat16-precision activations.  Every element enters the arithmetic as its
 * exact f32 value, so a call with F16 or BF16 x gives bit for bit the result of the
 * F32 call on those values converted to f32.
 */
typedef enum {
    Q2_0_ACT_F32 = 0,    /* IEEE single, 4-byte aligned */
    Q2_0_ACT_F16 = 1,    /* IEEE half, 2-byte aligned */
    Q2_0_ACT_BF16 = 2    /* bfloat16 (the upper 16 bits of an IEEE single), 2-byte aligned */
} q2_0_act_type;

/*
 * get_rows: gather rows of a Q2_0 matrix and dequantize them to f32
 * (bisque.today "WebGPU: add Q2_0 support", the paragraph on its three shaders:
 * the gather shader expands each selected row to f32, one block of 64 at a time).
 *   w      : M x K Q2_0 matrix (layout above), 2-byte aligned.
 *   ids    : n_ids int32 row indices, device memory, 4-byte aligned.
 *   out    : n_ids rows of K floats; row r starts at out + r*ld_out (ld_out >= K).
 * out[r][k] is the IEEE f32 product f32(q - 1) * f32(d) of weight k of row
 * ids[r] -- bit-exact, zero signs included.  An id outside [0, M) fills its row's
 * first K floats with quiet NaN and reads nothing.  Columns K..ld_out-1 are not
 * written.
 */
int q2_0_get_rows(const void *w, int64_t M, int64_t K, const int32_t *ids, int64_t n_ids,
                  float *out, int64_t ld_out, void *stream);

/*
 * mul_mat_vec: y = W x for 1 <= N <= 8 activation columns, fp32-grade
 * (bisque.today "WebGPU: add Q2_0 support", the matrix-vector paragraph: each
 * block's sum of (q - 1) * x is formed first and the scale applied once).
 *   w : M x K Q2_0 matrix, 2-byte aligned (16-byte aligned rows take the fast path).
 *   x : N columns of K floats at x + n*ldx, ldx >= K, 4-byte aligned.
 *   y : N columns of M floats at y + n*ldy, ldy >= M, 4-byte aligned; y[n][m] is
 *       overwritten.  x and y must not overlap.
 * Accuracy.  With A = sum_k |W[m][k] * x[n][k]|: y is exactly 0 where A is 0, and
 *     |y - y_exact| <= 1e-5 * A
 * for finite inputs with |x| < 2^100 and K <= 16384 whenever
 *     max_k |x[n][k]| * sum_k |W[m][k]| <= 2^21 * A          (range condition).
 * Why the condition: products are exact and sums f32, but x enters the matrix cores
 * in a form whose absolute error is tied to the largest activation near it.  For
 * N = 1 each 64-element block is scaled by a power of two and split into four 11-bit
 * fixed-point limbs (elements within 2^20 of the block's largest |x| are exact, the
 * others err by at most 2^-44 of it); otherwise each column is scaled by a power of
 * two and carried as an fp16 hi/lo pair (2^-22 relative error for elements within
 * 2^17 of the column's largest |x|, at most 2^-39 of that largest |x| below).  The
 * bound can therefore fail only where A is carried by activations some 2^21 below a
 * larger one that meets zero weights.  q2_0_mul_mat with Q2_0_PREC_F32 has no range
 * condition.
 * N > 8 returns Q2_0_ERR_UNSUPPORTED (use q2_0_mul_mat).
 */
int q2_0_mul_mat_vec(const void *w, int64_t M, int64_t K, const float *x, int64_t ldx, int64_t N,
                     float *y, int64_t ldy, void *stream);

/* One matrix of a grouped mat-vec (see q2_0_mul_mat_vec_group). */
typedef struct {
    const void *w;   /* M x K Q2_0 matrix (device), 2-byte aligned */
    int64_t M;       /* rows; 0 is allowed and writes nothing */
    float *y;        /* device: N columns of M floats at y + n*ldy, 4-byte aligned */
    int64_t ldy;     /* >= M */
} q2_0_mat_vec_item;

/*
 * mul_mat_vec_group: several mat-vecs that share K and the activation x, in as
 * few launches as possible: y_i = W_i x for i < n_items (for example the q, k and
 * v projections of one layer, or gate and up).  Same arithmetic, accuracy and
 * layouts as q2_0_mul_mat_vec; each y_i meets the same bound, and is deterministic
 * run to run (its last bits may depend on how items are grouped).
 *   items  : HOST array of n_items descriptors; read during the call only.
 *   x, ldx, N, stream: as for q2_0_mul_mat_vec (1 <= N <= 8).
 * The y_i must not overlap each other or x.  Errors are those of
 * q2_0_mul_mat_vec, checked for every item before anything is launched
 * (NULL also for items == NULL with n_items > 0); n_items < 0 is SHAPE.
 */
int q2_0_mul_mat_vec_group(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K,
                           const float *x, int64_t ldx, int64_t N, void *stream);

/* One product of a batched mat-vec (see q2_0_mul_mat_vec_batch). */
typedef struct {
    const void *w;   /* M x K Q2_0 matrix (device), 2-byte aligned */
    int64_t M;       /* rows; 0 is allowed and writes nothing */
    int64_t K;       /* a positive multiple of 64 */
    const void *x;   /* device activations of the call's x_type: N columns of K at x + n*ldx */
    int64_t ldx;     /* >= K, in elements */
    float *y;        /* device: N columns of M floats at y + n*ldy, 4-byte aligned */
    int64_t ldy;     /* >= M */
} q2_0_mat_vec_batch_item;

/*
 * mul_mat_vec_batch: y_i = W_i x_i for i < n_items, each item with its own K and
 * activation, in as few launches as possible -- for example every matrix a decode step
 * streams, whatever activation each reads.  Same arithmetic, accuracy and layouts as
 * q2_0_mul_mat_vec for every item.  Consecutive items with the same x, ldx and K share
 * one staging of x; one launch takes up to 64 items in up to 8 such runs (N <= 2; one run
 * for N > 2).  Results are deterministic run to run; their last bits may depend on how
 * items are grouped (the split of the work changes the order of f32 additions).
 *   items  : HOST array of n_items descriptors; read during the call only.
 *   x_type : a q2_0_act_type, for every item; 1 <= N <= 8 columns for every item.
 * The y_i must not overlap each other or any x_j.  Errors are those of
 * q2_0_mul_mat_vec_act, checked for every item before anything is launched (NULL also
 * for items == NULL with n_items > 0; n_items < 0 is SHAPE).
 */
int q2_0_mul_mat_vec_batch(const q2_0_mat_vec_batch_item *items, int64_t n_items, int x_type, int64_t N,
                           void *stream);

/*
 * mul_mat: y = W x for any N (batched prefill GEMM).
 * (bisque.today "WebGPU: add Q2_0 support", the paragraph on its three shaders:
 * its tiled GEMM expands the codes to fp16 weights in workgroup memory, sixteen
 * per thread.)
 *   Layouts and alignment as for q2_0_mul_mat_vec; precision is a q2_0_precision.
 *   Q2_0_PREC_F16_MFMA (fast):
 *     N <= 8 runs the mat-vec: its fp32-grade bound under its range condition.
 *     N > 8 forms the weights as fp16 d*(q-1), which is exact for |d| <= 32752,
 *     rounds x to fp16 (nearest-even) after scaling each column by a power of two
 *     that puts its max |x| in [2^14, 2^15) (undone exactly on the results), and
 *     accumulates in f32 on the matrix cores.  An element then errs by at most
 *     2^-11 of itself (within 2^28 of the column's largest |x|) or 2^-39 of that
 *     largest |x| (below), so with A = sum_k |W[m][k] x[n][k]|:
 *         |y - y_exact| <= 2e-3 * A
 *     for finite x with |x| < 2^100, |d| <= 32752 and K <= 16384 whenever
 *         max_k |x[n][k]| * sum_k |W[m][k]| <= 2^28 * A     (range condition).
 *   Q2_0_PREC_F32 (the accuracy fallback), any N: W as f32 (q-1) with d apart, x in
 *     f32, f32 fused multiply-adds of at most 64 terms per block sum (fp64 across
 *     blocks for N > 8): |y - y_exact| <= 1e-5 * A for all finite inputs whose
 *     products stay finite in f32, with no range condition (a weight of zero
 *     contributes exactly nothing); y is exactly 0 where A is 0.
 *   Q2_0_PREC_F32_MFMA (fp32-grade on the matrix cores):
 *     N <= 8 runs the mat-vec, as Q2_0_PREC_F16_MFMA does.
 *     N > 8 forms the weights as fp16 d*(q-1) (exact for |d| <= 32752), scales each
 *     column of x by the power of two that puts its max |x| in [2^14, 2^15) and
 *     carries every element as an fp16 pair hi = fp16(x), lo = fp16(x - hi) (2^-22
 *     relative error within 2^17 of the column's largest |x|, at most 2^-39 of that
 *     largest |x| below).  Both halves meet the weights on the matrix cores (products
 *     exact); every two 64-weight blocks are summed in an f32 accumulator of their own
 *     (8 matrix-core steps) and these sums are added in fp64.  Then
 *         |y - y_exact| <= 1e-5 * A
 *     for finite x with |x| < 2^100, |d| <= 32752 and K <= 16384 whenever
 *         max_k |x[n][k]| * sum_k |W[m][k]| <= 2^21 * A     (range condition),
 *     the mat-vec's condition; y is exactly 0 where A is 0.
 *   workspace / ws_bytes: device scratch the caller provides, 16-byte aligned, at
 *   least q2_0_mul_mat_workspace_bytes(M, K, N, precision) bytes: for
 *   Q2_0_PREC_F16_MFMA with N > 8, x as fp16 (N*K*2) and N column exponents, plus,
 *   when the output tile grid is too small to fill the GPU, the f32 partial sums of a
 *   K split (splits*N*M*4, split count <= 8, added in a fixed order); for
 *   Q2_0_PREC_F32_MFMA with N > 8 the same with x as two fp16 halves (2*N*K*2);
 *   otherwise 0 (then workspace may be NULL).
 *   Its contents are overwritten; it must not overlap w, x or y.
 */
int q2_0_mul_mat(const void *w, int64_t M, int64_t K, const float *x, int64_t ldx, int64_t N,
                 float *y, int64_t ldy, int precision, void *workspace, size_t ws_bytes,
                 void *stream);

/* Workspace bytes q2_0_mul_mat needs for these sizes (0 when none, and for invalid sizes). */
size_t q2_0_mul_mat_workspace_bytes(int64_t M, int64_t K, int64_t N, int precision);

/*
 * mul_mat_noalloc: q2_0_mul_mat for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).  No
 * workspace argument and no allocation of any kind: the fp16 GEMM's scratch is a
 * static device array of Q2_0_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on
 * every GPU it runs on until the process ends.  Arguments, arithmetic, results and errors
 * are those of q2_0_mul_mat, plus Q2_0_ERR_TOO_LARGE (checked last, nothing launched)
 * when q2_0_mul_mat_workspace_bytes(M, K, N, precision) exceeds that size -- e.g. the
 * 4096 x 12288 down projection at N = 512 needs 46 MB.  Every call on one GPU uses the
 * same scratch: calls that overlap in time on one GPU (two streams, two threads) race
 * and must be serialized by the caller.
 */
#define Q2_0_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int q2_0_mul_mat_noalloc(const void *w, int64_t M, int64_t K, const float *x, int64_t ldx, int64_t N,
                         float *y, int64_t ldy, int precision, void *stream);

/*
 * mul_mat_group: several q2_0_mul_mat products that share K and the activation x,
 * y_i = W_i x (a prefill layer's q, k and v projections, or gate and up).  Same
 * arithmetic, accuracy, layouts and routing as q2_0_mul_mat for each item; with
 * Q2_0_PREC_F16_MFMA or Q2_0_PREC_F32_MFMA and N > 8, x is converted to fp16 (its
 * hi/lo pair) once for all items and their
 * tiles run in shared launches (up to 16 matrices each), so small matrices fill the
 * GPU together.  Each y_i does not depend on the other items or on the grouping.
 *   items  : HOST array of n_items descriptors {w, M, y, ldy} (q2_0_mat_vec_item);
 *            read during the call only.  M = 0 items are skipped.
 *   x, ldx, N, precision, stream: as for q2_0_mul_mat.
 *   workspace / ws_bytes: at least q2_0_mul_mat_group_workspace_bytes() bytes,
 *            16-byte aligned: x as fp16 and its column exponents once, plus, when the
 *            group's tile grid is too small to fill the GPU, every item's split-K
 *            partial sums.  Overwritten; must not overlap w, x or y.
 * The y_i must not overlap each other or x.  Errors are those of q2_0_mul_mat,
 * checked for every item before anything is launched (NULL also for items == NULL
 * with n_items > 0; n_items < 0 is SHAPE).
 */
int q2_0_mul_mat_group(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K, const float *x,
                       int64_t ldx, int64_t N, int precision, void *workspace, size_t ws_bytes,
                       void *stream);

/* Workspace bytes q2_0_mul_mat_group needs (0 when none, and for invalid arguments). */
size_t q2_0_mul_mat_group_workspace_bytes(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K,
                                          int64_t N, int precision);

/*
 * The same four products with activations of element type x_type (a q2_0_act_type):
 * x points at N columns of K elements of that type, column n at element n*ldx
 * (ldx >= K), aligned to the element size.  Everything else -- w, y, items,
 * precision, routing, accuracy, workspace (the *_workspace_bytes queries above hold
 * for every x_type) and errors -- is that of the F32 call.  An unknown x_type
 * returns Q2_0_ERR_UNSUPPORTED, checked before alignment (which depends on it).
 * q2_0_mul_mat_vec(...) is q2_0_mul_mat_vec_act(..., Q2_0_ACT_F32, ...), and so on.
 */
int q2_0_mul_mat_vec_act(const void *w, int64_t M, int64_t K, const void *x, int x_type, int64_t ldx,
                         int64_t N, float *y, int64_t ldy, void *stream);
int q2_0_mul_mat_vec_group_act(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K, const void *x,
                               int x_type, int64_t ldx, int64_t N, void *stream);
int q2_0_mul_mat_act(const void *w, int64_t M, int64_t K, const void *x, int x_type, int64_t ldx, int64_t N,
                     float *y, int64_t ldy, int precision, void *workspace, size_t ws_bytes, void *stream);
int q2_0_mul_mat_group_act(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K, const void *x,
                           int x_type, int64_t ldx, int64_t N, int precision, void *workspace,
                           size_t ws_bytes, void *stream);

/*
 * mul_mat_id: the expert ("mixture of experts") product, which the WebGPU backend of
 * bisque.today "WebGPU: add Q2_0 support" leaves out for Q2_0 (the paragraph on what
 * the change does not cover).  For token t < n_tokens and slot u < n_used:
 *     y[t][u] = W_{ids[t][u]} x[t][u mod x_slots]
 * with W_e the e-th of n_expert M x K Q2_0 matrices.
 *   w       : n_expert matrices back to back (device), expert e at byte
 *             e*M*(K/64)*18, 2-byte aligned (16-byte aligned rows are faster).
 *   x       : activations of element type x_type (a q2_0_act_type); column (t, s)
 *             for s < x_slots at element (t*x_slots + s)*ldx, ldx >= K.  x_slots is 1
 *             (every slot of a token multiplies the token's activation, like an
 *             expert layer's gate and up projections) or n_used (one activation per
 *             slot, like its down projection).
 *   ids     : DEVICE int32 [n_tokens][n_used] expert indices, 4-byte aligned.  An id
 *             outside [0, n_expert) makes its y column quiet NaN and reads nothing.
 *   y       : f32 column (t, u) at y + (t*n_used + u)*ldy, ldy >= M.
 *   precision: as for q2_0_mul_mat: Q2_0_PREC_F16_MFMA (x rounded to fp16 as there,
 *             2e-3 bound under its range condition; few pairs -- n_tokens <= 8, or
 *             fewer pairs than twice n_expert -- take the fp32-grade mat-vec, one per
 *             pair, with the mat-vec's bound and range condition: it streams the
 *             experts faster than the GEMM decodes them while experts get about two
 *             pairs or fewer) or Q2_0_PREC_F32 (the fp32 GEMM, 1e-5 bound, no range
 *             condition); Q2_0_PREC_F32_MFMA runs as Q2_0_PREC_F32, whose guarantee
 *             covers its own.
 *   workspace / ws_bytes: at least q2_0_mul_mat_id_workspace_bytes() bytes, 16-byte
 *             aligned: the routing tables (the pairs sorted by expert, stably) and,
 *             for Q2_0_PREC_F16_MFMA, x as fp16 in expert order.  Overwritten.
 * The routing runs on the GPU; the result does not depend on timing or on how the
 * pairs fall to the experts beyond the products themselves.
 * Errors: SHAPE (also n_expert < 1 or > 8192, n_tokens*n_used > 2^20, x_slots not 1
 * or n_used), the no-op for M == 0 or no pairs, NULL, LAYOUT, UNSUPPORTED (unknown
 * x_type, checked before alignment, or precision), ALIGN, WORKSPACE.
 */
int q2_0_mul_mat_id(const void *w, int64_t n_expert, int64_t M, int64_t K, const void *x, int x_type,
                    int64_t ldx, int64_t x_slots, const int32_t *ids, int64_t n_used, int64_t n_tokens,
                    float *y, int64_t ldy, int precision, void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes q2_0_mul_mat_id needs (0 for invalid sizes). */
size_t q2_0_mul_mat_id_workspace_bytes(int64_t n_expert, int64_t M, int64_t K, int64_t n_used, int64_t n_tokens,
                                       int precision);

/*
 * quantize: f32 weights -> Q2_0 by the reference quantizer (aisvetem.cz, "Llama.cpp
 * umi dvoubitovy Q2_0 i na kartach NVIDIA", section "Na bezny model to neni": the
 * block's largest |w| is the scale and each weight goes to the nearest level).
 * Per block of 64: d = max|w| rounded to the nearest half (ties to even; at or
 * above 65520 it is +inf); each weight takes the nearest of -d, 0, d, 2d, a weight
 * exactly between two levels the one nearer zero; a block whose d is 0 (or inf) is
 * code 1 everywhere.  Code 3 is therefore never produced.
 *   src   : M rows of K floats (device), row m at src + m*ld_src, ld_src >= K,
 *           4-byte aligned; finite values (NaN / inf inputs are out of contract).
 *   w     : M x K Q2_0 output (device, layout above), 2-byte aligned; must not
 *           overlap src.
 * Errors: SHAPE, the M == 0 no-op, NULL, LAYOUT (ld_src < K), ALIGN.
 */
int q2_0_quantize(const float *src, int64_t M, int64_t K, int64_t ld_src, void *w, void *stream);

/*
 * repack_g128: the older group-128 packing (34 bytes per 128 weights; aisvetem.cz,
 * same article, sections "Sest procent, o ktera se vedl spor" and the closing
 * paragraph on the two kinds of files) -> Q2_0 with group 64, losslessly.  Read as
 * the group-64 block extended: a little-endian half scale d, then eight
 * little-endian 32-bit words, code i of word w belonging to weight 16w+i.  Legacy
 * block j of a row becomes blocks 2j and 2j+1 of the output row, both with scale d,
 * holding words 0..3 and 4..7.
 *   w128  : M rows of K/128 legacy blocks (device), row m at byte m*(K/128)*34,
 *           2-byte aligned.
 *   w     : M x K Q2_0 output (device), 2-byte aligned; must not overlap w128.
 * Errors: SHAPE (also K % 128 != 0), the M == 0 no-op, NULL, ALIGN.
 */
int q2_0_repack_g128(const void *w128, int64_t M, int64_t K, void *w, void *stream);

/* A static, human-readable name for a status code. */
const char *q2_0_status_string(int status);

/* The hipError_t of the last Q2_0_ERR_HIP returned on the calling thread (0 if none). */
int q2_0_last_hip_error(void);

/* Library version string, e.g. "q2_0 0.1.0 gfx950". */
const char *q2_0_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q2_0_H */
