// C ABI of libq2_0.so: argument validation and dispatch.  Declared in include/q2_0.h.
//
// Validation runs entirely on the host and returns before any HIP call, so a bad
// argument never reaches a kernel.  The kernels themselves assume what is checked
// here: K a positive multiple of 64, strides at least the row length, 2-byte
// aligned weights, 4-byte aligned floats and ids, and sizes within the grid limits.
#include "../../include/q2_0.h"
#include "q2_0_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

// Largest sizes the launch geometry covers (grid.y limit times the tile, and
// 32-bit in-row offsets).
constexpr int64_t kMaxK = (int64_t)1 << 24;          // 16 Mi weights per row
constexpr int64_t kMaxRows = ((int64_t)1 << 31) - 1;  // M and n_ids
constexpr int64_t kMaxGemmN = (int64_t)65535 * 64;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return Q2_0_OK;
    g_last_hip_error = (int)e;
    return Q2_0_ERR_HIP;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool known_precision(int p) { return p == Q2_0_PREC_F16_MFMA || p == Q2_0_PREC_F32 || p == Q2_0_PREC_F32_MFMA; }

int check_shape(int64_t M, int64_t K, int64_t N) {
    if (K <= 0 || K % Q2_0_BLOCK_WEIGHTS != 0 || K > kMaxK) return Q2_0_ERR_SHAPE;
    if (M < 0 || N < 0 || M > kMaxRows) return Q2_0_ERR_SHAPE;
    return Q2_0_OK;
}

// Common checks of the products after the empty no-op: NULL, LAYOUT, then the
// activation type (alignment depends on it) and ALIGN.
int check_product(const void *w, int64_t M, int64_t K, const void *x, int x_type, int64_t ldx,
                  const float *y, int64_t ldy) {
    if (!w || !x || !y) return Q2_0_ERR_NULL;
    if (ldx < K || ldy < M) return Q2_0_ERR_LAYOUT;
    if (x_type != Q2_0_ACT_F32 && x_type != Q2_0_ACT_F16 && x_type != Q2_0_ACT_BF16) return Q2_0_ERR_UNSUPPORTED;
    if (!aligned(w, 2) || !aligned(x, q2_0::act_bytes((q2_0::Act)x_type)) || !aligned(y, 4)) return Q2_0_ERR_ALIGN;
    return Q2_0_OK;
}

int mul_mat_vec_impl(const void *w, int64_t M, int64_t K, const void *x, int x_type, int64_t ldx, int64_t N,
                     float *y, int64_t ldy, void *stream) {
    int st = check_shape(M, K, N);
    if (st) return st;
    if (M == 0 || N == 0) return Q2_0_OK;
    st = check_product(w, M, K, x, x_type, ldx, y, ldy);
    if (st) return st;
    if (N > Q2_0_MAT_VEC_MAX_N) return Q2_0_ERR_UNSUPPORTED;
    return hip_status(q2_0::launch_mat_vec(static_cast<const uint8_t *>(w), M, (int)(K / Q2_0_BLOCK_WEIGHTS), x,
                                           (q2_0::Act)x_type, ldx, (int)N, y, ldy,
                                           static_cast<hipStream_t>(stream)));
}

int mul_mat_vec_group_impl(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K, const void *x,
                           int x_type, int64_t ldx, int64_t N, void *stream) {
    int st = check_shape(0, K, N);
    if (st) return st;
    if (n_items < 0) return Q2_0_ERR_SHAPE;
    if (n_items == 0 || N == 0) return Q2_0_OK;
    if (!items) return Q2_0_ERR_NULL;
    for (int64_t i = 0; i < n_items; ++i) {
        st = check_shape(items[i].M, K, N);
        if (st) return st;
    }
    bool any = false;
    for (int64_t i = 0; i < n_items; ++i) {
        if (items[i].M == 0) continue;
        any = true;
        st = check_product(items[i].w, items[i].M, K, x, x_type, ldx, items[i].y, items[i].ldy);
        if (st) return st;
    }
    if (!any) return Q2_0_OK;
    if (N > Q2_0_MAT_VEC_MAX_N) return Q2_0_ERR_UNSUPPORTED;
    return hip_status(q2_0::launch_mat_vec_group(items, n_items, (int)(K / Q2_0_BLOCK_WEIGHTS), x,
                                                 (q2_0::Act)x_type, ldx, (int)N,
                                                 static_cast<hipStream_t>(stream)));
}

int mul_mat_vec_batch_impl(const q2_0_mat_vec_batch_item *items, int64_t n_items, int x_type, int64_t N,
                           void *stream) {
    if (n_items < 0 || N < 0) return Q2_0_ERR_SHAPE;
    if (n_items > 0 && !items) return Q2_0_ERR_NULL;
    for (int64_t i = 0; i < n_items; ++i) {
        const int st = check_shape(items[i].M, items[i].K, N);
        if (st) return st;
    }
    bool any = false;
    for (int64_t i = 0; i < n_items && N > 0; ++i) {
        if (items[i].M == 0) continue;
        any = true;
        const int st = check_product(items[i].w, items[i].M, items[i].K, items[i].x, x_type, items[i].ldx,
                                     items[i].y, items[i].ldy);
        if (st) return st;
    }
    if (!any) return Q2_0_OK;
    if (N > Q2_0_MAT_VEC_MAX_N) return Q2_0_ERR_UNSUPPORTED;
    return hip_status(q2_0::launch_mat_vec_batch(items, n_items, (q2_0::Act)x_type, (int)N,
                                                 static_cast<hipStream_t>(stream)));
}

int mul_mat_impl(const void *w, int64_t M, int64_t K, const void *x, int x_type, int64_t ldx, int64_t N,
                 float *y, int64_t ldy, int precision, void *workspace, size_t ws_bytes, void *stream);
int mul_mat_group_impl(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K, const void *x, int x_type,
                       int64_t ldx, int64_t N, int precision, void *workspace, size_t ws_bytes, void *stream);

}  // namespace

extern "C" {

int q2_0_get_rows(const void *w, int64_t M, int64_t K, const int32_t *ids, int64_t n_ids,
                  float *out, int64_t ld_out, void *stream) {
    int st = check_shape(M, K, 0);
    if (st) return st;
    if (n_ids < 0 || n_ids > kMaxRows) return Q2_0_ERR_SHAPE;
    if (n_ids == 0) return Q2_0_OK;
    if (!w || !ids || !out) return Q2_0_ERR_NULL;
    if (ld_out < K) return Q2_0_ERR_LAYOUT;
    if (!aligned(w, 2) || !aligned(ids, 4) || !aligned(out, 4)) return Q2_0_ERR_ALIGN;
    return hip_status(q2_0::launch_get_rows(static_cast<const uint8_t *>(w), M,
                                            (int)(K / Q2_0_BLOCK_WEIGHTS), ids, n_ids, out, ld_out,
                                            static_cast<hipStream_t>(stream)));
}

int q2_0_mul_mat_vec(const void *w, int64_t M, int64_t K, const float *x, int64_t ldx, int64_t N,
                     float *y, int64_t ldy, void *stream) {
    return mul_mat_vec_impl(w, M, K, x, Q2_0_ACT_F32, ldx, N, y, ldy, stream);
}

int q2_0_mul_mat_vec_act(const void *w, int64_t M, int64_t K, const void *x, int x_type, int64_t ldx,
                         int64_t N, float *y, int64_t ldy, void *stream) {
    return mul_mat_vec_impl(w, M, K, x, x_type, ldx, N, y, ldy, stream);
}

int q2_0_mul_mat_vec_group(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K,
                           const float *x, int64_t ldx, int64_t N, void *stream) {
    return mul_mat_vec_group_impl(items, n_items, K, x, Q2_0_ACT_F32, ldx, N, stream);
}

int q2_0_mul_mat_vec_group_act(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K, const void *x,
                               int x_type, int64_t ldx, int64_t N, void *stream) {
    return mul_mat_vec_group_impl(items, n_items, K, x, x_type, ldx, N, stream);
}

int q2_0_mul_mat_vec_batch(const q2_0_mat_vec_batch_item *items, int64_t n_items, int x_type, int64_t N,
                           void *stream) {
    return mul_mat_vec_batch_impl(items, n_items, x_type, N, stream);
}

size_t q2_0_mul_mat_workspace_bytes(int64_t M, int64_t K, int64_t N, int precision) {
    if (check_shape(M, K, N) || N > kMaxGemmN) return 0;
    if ((precision != Q2_0_PREC_F16_MFMA && precision != Q2_0_PREC_F32_MFMA) || N <= Q2_0_MAT_VEC_MAX_N) return 0;
    const q2_0_mat_vec_item item{nullptr, M, nullptr, M};
    // x as fp16 (hi/lo pairs for the fp32-grade GEMM) (+ split-K state)
    return q2_0::gemm_f16_workspace_bytes(&item, 1, K, N, precision == Q2_0_PREC_F32_MFMA);
}

int q2_0_mul_mat(const void *w, int64_t M, int64_t K, const float *x, int64_t ldx, int64_t N,
                 float *y, int64_t ldy, int precision, void *workspace, size_t ws_bytes,
                 void *stream) {
    return mul_mat_impl(w, M, K, x, Q2_0_ACT_F32, ldx, N, y, ldy, precision, workspace, ws_bytes, stream);
}

int q2_0_mul_mat_act(const void *w, int64_t M, int64_t K, const void *x, int x_type, int64_t ldx, int64_t N,
                     float *y, int64_t ldy, int precision, void *workspace, size_t ws_bytes, void *stream) {
    return mul_mat_impl(w, M, K, x, x_type, ldx, N, y, ldy, precision, workspace, ws_bytes, stream);
}

size_t q2_0_mul_mat_group_workspace_bytes(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K,
                                          int64_t N, int precision) {
    if (check_shape(0, K, N) || N > kMaxGemmN || n_items < 0 || (n_items > 0 && !items)) return 0;
    if ((precision != Q2_0_PREC_F16_MFMA && precision != Q2_0_PREC_F32_MFMA) || N <= Q2_0_MAT_VEC_MAX_N ||
        n_items == 0)
        return 0;
    for (int64_t i = 0; i < n_items; ++i)
        if (check_shape(items[i].M, K, N)) return 0;
    return q2_0::gemm_f16_workspace_bytes(items, n_items, K, N, precision == Q2_0_PREC_F32_MFMA);
}

int q2_0_mul_mat_group(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K, const float *x,
                       int64_t ldx, int64_t N, int precision, void *workspace, size_t ws_bytes, void *stream) {
    return mul_mat_group_impl(items, n_items, K, x, Q2_0_ACT_F32, ldx, N, precision, workspace, ws_bytes,
                              stream);
}

int q2_0_mul_mat_group_act(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K, const void *x,
                           int x_type, int64_t ldx, int64_t N, int precision, void *workspace,
                           size_t ws_bytes, void *stream) {
    return mul_mat_group_impl(items, n_items, K, x, x_type, ldx, N, precision, workspace, ws_bytes, stream);
}

}  // extern "C"

namespace {

constexpr int64_t kMaxExperts = 8192;
constexpr int64_t kMaxPairs = (int64_t)1 << 20;

int check_moe_shape(int64_t n_expert, int64_t M, int64_t K, int64_t n_used, int64_t n_tokens, int precision) {
    int st = check_shape(M, K, 0);
    if (st) return st;
    if (n_expert < 1 || n_expert > kMaxExperts || n_used < 0 || n_tokens < 0) return Q2_0_ERR_SHAPE;
    if (n_used > kMaxPairs || n_tokens > kMaxPairs || n_used * n_tokens > kMaxPairs) return Q2_0_ERR_SHAPE;
    const int64_t n_pairs = n_used * n_tokens;
    // launch grids: the fp32 path has one workgroup row per tile-list entry (grid.y)
    if (precision == Q2_0_PREC_F32 && q2_0::moe_max_tiles(n_expert, n_pairs, 64) > 65535) return Q2_0_ERR_SHAPE;
    if ((M + 127) / 128 * q2_0::moe_max_tiles(n_expert, n_pairs, 64) > kMaxRows) return Q2_0_ERR_SHAPE;
    return Q2_0_OK;
}

int moe_tile_w(int) { return 64; }   // column tile of both expert GEMMs

}  // namespace

extern "C" {

size_t q2_0_mul_mat_id_workspace_bytes(int64_t n_expert, int64_t M, int64_t K, int64_t n_used, int64_t n_tokens,
                                       int precision) {
    if (precision == Q2_0_PREC_F32_MFMA) precision = Q2_0_PREC_F32;   // the fp32 GEMM covers its guarantee
    if (check_moe_shape(n_expert, M, K, n_used, n_tokens, precision)) return 0;
    if (precision != Q2_0_PREC_F16_MFMA && precision != Q2_0_PREC_F32) return 0;
    const int64_t n_pairs = n_used * n_tokens;
    size_t b = q2_0::moe_route_bytes(n_expert, n_pairs, moe_tile_w(precision));
    if (precision == Q2_0_PREC_F16_MFMA) b += q2_0::gemm_f16_moe_scratch_bytes(K, n_pairs);
    return b;
}

int q2_0_mul_mat_id(const void *w, int64_t n_expert, int64_t M, int64_t K, const void *x, int x_type,
                    int64_t ldx, int64_t x_slots, const int32_t *ids, int64_t n_used, int64_t n_tokens,
                    float *y, int64_t ldy, int precision, void *workspace, size_t ws_bytes, void *stream) {
    if (precision == Q2_0_PREC_F32_MFMA) precision = Q2_0_PREC_F32;   // the fp32 GEMM covers its guarantee
    int st = check_moe_shape(n_expert, M, K, n_used, n_tokens, precision);
    if (st) return st;
    if (x_slots != 1 && x_slots != n_used) return Q2_0_ERR_SHAPE;
    const int64_t n_pairs = n_used * n_tokens;
    if (M == 0 || n_pairs == 0) return Q2_0_OK;
    if (!ids) return Q2_0_ERR_NULL;
    st = check_product(w, M, K, x, x_type, ldx, y, ldy);
    if (st) return st;
    if (!aligned(ids, 4)) return Q2_0_ERR_ALIGN;
    if (precision != Q2_0_PREC_F16_MFMA && precision != Q2_0_PREC_F32) return Q2_0_ERR_UNSUPPORTED;
    const size_t need = q2_0_mul_mat_id_workspace_bytes(n_expert, M, K, n_used, n_tokens, precision);
    if (ws_bytes < need || !workspace || !aligned(workspace, 16)) return Q2_0_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const int nb = (int)(K / Q2_0_BLOCK_WEIGHTS);
    const q2_0::Act xt = (q2_0::Act)x_type;
    // Few pairs with the fast precision: one fp32-grade mat-vec per pair -- up to 8 tokens
    // (as q2_0_mul_mat with N <= 8), and while the pairs are fewer than twice the experts.
    // The routed GEMM reads each used expert once but is bound by decoding the weights
    // (~1.6 TB/s of weight bytes); the per-pair mat-vec reads an expert once per pair but
    // streams at ~4 TB/s, so it wins while the pairs number under about 2.5 times the
    // distinct experts, whatever M and K.  Measured on 128 experts of 768 x 2048, 8 slots:
    // 9, 16 and 32 tokens 14.8, 20.5 and 34.5 us per call against 27.7, 28.7 and 36.5 for
    // the GEMM; 48 tokens 48.2 against 35.9.
    const bool few_pairs = n_tokens <= Q2_0_MAT_VEC_MAX_N || n_pairs < 2 * n_expert;
    if (precision == Q2_0_PREC_F16_MFMA && few_pairs && n_pairs <= 65535 &&
        q2_0::mat_vec_mfma_eligible(wb, M, nb, x, xt, ldx)) {
        // (out-of-range ids: NaN columns, written by the same launch)
        return hip_status(q2_0::launch_mat_vec_mfma_pairs(wb, M, nb, x, xt, ldx, ids, (int)n_expert, (int)n_used,
                                                          (int)x_slots, (int)n_pairs, y, ldy, s));
    }
    q2_0::MoeRoute r;
    // the fp16 GEMM's scratch follows the routing tables; where it can, the routing launch
    // also converts x into it
    void *scratch = static_cast<uint8_t *>(workspace) + q2_0::moe_route_bytes(n_expert, n_pairs, moe_tile_w(precision));
    const bool fused = precision == Q2_0_PREC_F16_MFMA && q2_0::moe_route_converts((int)n_expert);
    if (fused)
        st = hip_status(q2_0::launch_moe_route_convert(ids, (int)n_pairs, (int)n_expert, (int)n_used, (int)x_slots,
                                                       moe_tile_w(precision), workspace, &r, x, xt, ldx, (int)K,
                                                       scratch, s));
    else
        st = hip_status(q2_0::launch_moe_route(ids, (int)n_pairs, (int)n_expert, (int)n_used, (int)x_slots,
                                               moe_tile_w(precision), workspace, &r, s));
    if (st) return st;
    if (precision == Q2_0_PREC_F16_MFMA)   // (its launch also fills the out-of-range pairs' columns)
        return hip_status(q2_0::launch_gemm_f16_moe(wb, M, nb, x, xt, ldx, r, y, ldy, scratch, s, fused));
    st = hip_status(q2_0::launch_gemm_f32_moe(wb, M, nb, x, xt, ldx, r, y, ldy, s));
    if (st) return st;
    return hip_status(q2_0::launch_moe_fill_bad(r, M, y, ldy, s));
}

int q2_0_quantize(const float *src, int64_t M, int64_t K, int64_t ld_src, void *w, void *stream) {
    int st = check_shape(M, K, 0);
    if (st) return st;
    if (M == 0) return Q2_0_OK;
    if (!src || !w) return Q2_0_ERR_NULL;
    if (ld_src < K) return Q2_0_ERR_LAYOUT;
    if (!aligned(src, 4) || !aligned(w, 2)) return Q2_0_ERR_ALIGN;
    return hip_status(q2_0::launch_quantize(src, M, (int)(K / Q2_0_BLOCK_WEIGHTS), ld_src,
                                            static_cast<uint8_t *>(w), static_cast<hipStream_t>(stream)));
}

int q2_0_repack_g128(const void *w128, int64_t M, int64_t K, void *w, void *stream) {
    int st = check_shape(M, K, 0);
    if (st) return st;
    if (K % 128 != 0) return Q2_0_ERR_SHAPE;
    if (M == 0) return Q2_0_OK;
    if (!w128 || !w) return Q2_0_ERR_NULL;
    if (!aligned(w128, 2) || !aligned(w, 2)) return Q2_0_ERR_ALIGN;
    return hip_status(q2_0::launch_repack_g128(static_cast<const uint8_t *>(w128), M, K, static_cast<uint8_t *>(w),
                                               static_cast<hipStream_t>(stream)));
}

const char *q2_0_status_string(int status) {
    switch (status) {
        case Q2_0_OK: return "Q2_0_OK";
        case Q2_0_ERR_NULL: return "Q2_0_ERR_NULL: a required pointer is NULL";
        case Q2_0_ERR_SHAPE: return "Q2_0_ERR_SHAPE: K must be a positive multiple of 64 and sizes non-negative and within limits";
        case Q2_0_ERR_LAYOUT: return "Q2_0_ERR_LAYOUT: a leading dimension is smaller than the row length";
        case Q2_0_ERR_ALIGN: return "Q2_0_ERR_ALIGN: w must be 2-byte aligned and other buffers aligned to their element size";
        case Q2_0_ERR_UNSUPPORTED: return "Q2_0_ERR_UNSUPPORTED: N > 8 for mat-vec, or unknown precision or activation type";
        case Q2_0_ERR_WORKSPACE: return "Q2_0_ERR_WORKSPACE: workspace missing, too small or not 16-byte aligned";
        case Q2_0_ERR_HIP: return "Q2_0_ERR_HIP: a HIP launch failed";
        case Q2_0_ERR_TOO_LARGE:
            return "Q2_0_ERR_TOO_LARGE: the call needs more scratch than Q2_0_NOALLOC_SCRATCH_BYTES";
        default: return "unknown q2_0 status";
    }
}

int q2_0_last_hip_error(void) { return g_last_hip_error; }

const char *q2_0_version(void) { return "q2_0 0.1.0 gfx950"; }

}  // extern "C"

namespace {

}  // namespace

namespace q2_0 {

int record_hip_error(hipError_t e) { return hip_status(e); }

// Every check of q2_0_mul_mat but the workspace one; *noop is set for the empty no-op.
int check_mul_mat(const void *w, int64_t M, int64_t K, const void *x, int x_type, int64_t ldx, int64_t N,
                  const float *y, int64_t ldy, int precision, bool *noop) {
    *noop = false;
    int st = check_shape(M, K, N);
    if (st) return st;
    if (N > kMaxGemmN) return Q2_0_ERR_SHAPE;
    if (((M + 127) / 128) * ((N + 127) / 128) * 8 > kMaxRows) return Q2_0_ERR_SHAPE;   // launch grid
    if (M == 0 || N == 0) {
        *noop = true;
        return Q2_0_OK;
    }
    st = check_product(w, M, K, x, x_type, ldx, y, ldy);
    if (st) return st;
    if (!known_precision(precision)) return Q2_0_ERR_UNSUPPORTED;
    return Q2_0_OK;
}

}  // namespace q2_0

namespace {

int mul_mat_impl(const void *w, int64_t M, int64_t K, const void *x, int x_type, int64_t ldx, int64_t N,
                 float *y, int64_t ldy, int precision, void *workspace, size_t ws_bytes, void *stream) {
    bool noop;
    const int st = q2_0::check_mul_mat(w, M, K, x, x_type, ldx, N, y, ldy, precision, &noop);
    if (st || noop) return st;
    const size_t need = q2_0_mul_mat_workspace_bytes(M, K, N, precision);
    if (ws_bytes < need || (need && (!workspace || !aligned(workspace, 16)))) return Q2_0_ERR_WORKSPACE;
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const int nb = (int)(K / Q2_0_BLOCK_WEIGHTS);
    const q2_0::Act xt = (q2_0::Act)x_type;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (precision == Q2_0_PREC_F32) {
        // the accuracy fallback: f32 arithmetic, no condition on the activations' range
        if (N <= Q2_0_MAT_VEC_MAX_N) return hip_status(q2_0::launch_mat_vec_f32(wb, M, nb, x, xt, ldx, (int)N, y, ldy, s));
        return hip_status(q2_0::launch_gemm_f32(wb, M, nb, x, xt, ldx, N, y, ldy, s));
    }
    if (N <= Q2_0_MAT_VEC_MAX_N)
        return hip_status(q2_0::launch_mat_vec(wb, M, nb, x, xt, ldx, (int)N, y, ldy, s));
    const q2_0_mat_vec_item m{w, M, y, ldy};
    return hip_status(
        q2_0::launch_gemm_f16_group(&m, 1, nb, x, xt, ldx, N, workspace, s, precision == Q2_0_PREC_F32_MFMA));
}

int mul_mat_group_impl(const q2_0_mat_vec_item *items, int64_t n_items, int64_t K, const void *x, int x_type,
                       int64_t ldx, int64_t N, int precision, void *workspace, size_t ws_bytes, void *stream) {
    int st = check_shape(0, K, N);
    if (st) return st;
    if (N > kMaxGemmN || n_items < 0) return Q2_0_ERR_SHAPE;
    if (n_items == 0 || N == 0) return Q2_0_OK;
    if (!items) return Q2_0_ERR_NULL;
    int64_t row_tiles = 0;
    for (int64_t i = 0; i < n_items; ++i) {
        st = check_shape(items[i].M, K, N);
        if (st) return st;
        row_tiles += (items[i].M + 127) / 128;
    }
    if (row_tiles * ((N + 127) / 128) * 8 > kMaxRows) return Q2_0_ERR_SHAPE;   // launch grid
    bool any = false;
    for (int64_t i = 0; i < n_items; ++i) {
        if (items[i].M == 0) continue;
        any = true;
        st = check_product(items[i].w, items[i].M, K, x, x_type, ldx, items[i].y, items[i].ldy);
        if (st) return st;
    }
    if (!any) return Q2_0_OK;
    if (!known_precision(precision)) return Q2_0_ERR_UNSUPPORTED;
    const size_t need = q2_0_mul_mat_group_workspace_bytes(items, n_items, K, N, precision);
    if (ws_bytes < need || (need && (!workspace || !aligned(workspace, 16)))) return Q2_0_ERR_WORKSPACE;
    const int nb = (int)(K / Q2_0_BLOCK_WEIGHTS);
    const q2_0::Act xt = (q2_0::Act)x_type;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (precision == Q2_0_PREC_F32) {
        for (int64_t i = 0; i < n_items; ++i) {
            if (items[i].M == 0) continue;
            const uint8_t *wi = static_cast<const uint8_t *>(items[i].w);
            st = hip_status(N <= Q2_0_MAT_VEC_MAX_N
                                ? q2_0::launch_mat_vec_f32(wi, items[i].M, nb, x, xt, ldx, (int)N, items[i].y,
                                                           items[i].ldy, s)
                                : q2_0::launch_gemm_f32(wi, items[i].M, nb, x, xt, ldx, N, items[i].y, items[i].ldy,
                                                        s));
            if (st) return st;
        }
        return Q2_0_OK;
    }
    if (N <= Q2_0_MAT_VEC_MAX_N)
        return hip_status(q2_0::launch_mat_vec_group(items, n_items, nb, x, xt, ldx, (int)N, s));
    return hip_status(
        q2_0::launch_gemm_f16_group(items, n_items, nb, x, xt, ldx, N, workspace, s, precision == Q2_0_PREC_F32_MFMA));
}

}  // namespace
