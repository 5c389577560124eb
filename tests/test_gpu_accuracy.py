"""GPU checks of the accuracy contracts in include/q2_0.h at their stated limits.

The fast paths carry x through the matrix cores in forms whose error is tied to the
largest activation near it, so their bounds hold under a range condition,
    max_k |x[n][k]| * sum_k |W[m][k]| <= 2^c * A[n][m],   A = sum_k |W[m][k] x[n][k]|,
with c = 21 for the mat-vec (1e-5) and c = 28 for the fp16 GEMM (2e-3).  The hardest
input inside the condition is a large activation that meets only zero weights (it adds
nothing to A): these tests put one at 0.9 of the limit, on every kernel path, and at the
magnitudes 1e4, 1e6 and 2^24.  Q2_0_PREC_F32 promises 1e-5 with no condition; it is
tested with zero-weighted activations up to 1e30.

Also here: the Qwen3-8B-shaped prefill calls that take a K split (o, 4096 x 4096 at
N = 512: two ways) or a three-matrix group (q/k/v) on sampled rows.
"""

import numpy as np
import pytest

import oracle
from ternary_bit_quantized_amd import q2_0 as B
from ternary_bit_quantized_amd import synth
from test_gpu_parity import (REL_F16, REL_F32, assert_products, dev, run_gemm_group, run_mat_vec,
                             run_mul_mat, ws)

pytestmark = pytest.mark.gpu

C_MAT_VEC = 21
C_GEMM_F16 = 28
K0_BLOCK, K0_OFF = 3, 17   # the zero-weighted column: block 3, element 17


def zero_column_case(seed, M, K, N):
    """Ternary W whose column k0 is code 1 (weight 0) in every row; x ~ N(0, 1) with x[:, k0]
    still 0; and min over rows and columns of A / sum|W| (the mean |x| the weights see)."""
    rng = synth.rng_for(40 + seed, M, K, N)
    codes = rng.integers(0, 3, size=(M, K), dtype=np.uint8)
    k0 = 64 * K0_BLOCK + K0_OFF
    codes[:, k0] = 1
    d = rng.uniform(0.005, 0.05, size=(M, K // 64)).astype(np.float16)
    w = synth.pack(codes, d)
    x = synth.activations(40 + seed, M, K, N, K)
    x[:, k0] = 0.0
    return w, x, k0


def rows_of(M):
    return None if M < 1000 else np.unique(np.concatenate([np.arange(0, M, 41), [M - 1]]))


def ratio_min(w, M, K, x, rows):
    """min over (n, m) of A[n][m] / sum_k |W[m][k]| on the checked rows."""
    _, A = oracle.mul_mat(w, M, K, x, rows=rows)
    _, S = oracle.mul_mat(w, M, K, np.ones((1, K), dtype=np.float32), rows=rows)
    return float(np.min(A / S))


def with_outlier(x, k0, big):
    x = x.copy()
    x[:, k0] = np.float32(big)
    return x


# ------------------------------------------------------------------ mat-vec (every kernel path)

# (M, K, N): the streaming kernels (M >= 16384) in limb mode (N = 1; K = 512 has a ragged
# half stage), hi/lo mode (N = 2) and the 16-row-tile kernel (N = 4, 8); the K-split
# kernel (M < 16384)
MV_PATHS = [(16400, 512, 1), (16400, 4096, 1), (16400, 12288, 1), (16400, 4096, 2), (16400, 12288, 2),
            (16400, 4096, 4), (16400, 2048, 8), (300, 4096, 1), (300, 4096, 4)]


@pytest.mark.parametrize("M,K,N", MV_PATHS)
def test_mat_vec_zero_weighted_outlier_at_the_limit(M, K, N):
    w, x, k0 = zero_column_case(1, M, K, N)
    rows = rows_of(M)
    limit = 2.0 ** C_MAT_VEC * ratio_min(w, M, K, x, rows)
    wd = dev(w)
    for big in (1e4, 1e6, 0.9 * limit, -0.9 * limit):
        if abs(big) > limit:
            continue
        xb = with_outlier(x, k0, big)
        y = run_mat_vec(wd, M, K, xb)
        assert_products(y, w, M, K, xb, REL_F32, rows=rows,
                        what="mat-vec M=%d K=%d N=%d outlier %.4g (limit %.4g)" % (M, K, N, big, limit))


def test_mat_vec_limbs_outlier_in_its_own_block():
    """N = 1 scales per 64-element block: an outlier far beyond the column condition, in a
    block whose weights are all zero, leaves every other block exact."""
    M, K = 16400, 4096
    w, x, k0 = zero_column_case(2, M, K, 1)
    codes_blk = np.ones((M, 64), dtype=np.uint8)
    d = np.full((M, 1), 0.01, dtype=np.float16)
    blk = synth.pack(codes_blk, d)                   # block K0_BLOCK: weight 0 everywhere
    w = w.copy()
    w[:, 18 * K0_BLOCK:18 * (K0_BLOCK + 1)] = blk
    xb = with_outlier(x, k0, 2.0 ** 60)
    y = run_mat_vec(dev(w), M, K, xb)
    assert_products(y, w, M, K, xb, REL_F32, rows=rows_of(M), what="limbs, outlier 2^60 in a zero block")


# ------------------------------------------------------------------ fp16-MFMA GEMM

@pytest.mark.parametrize("M,K,N", [(1024, 4096, 64), (256, 12288, 16), (300, 2048, 130)])
def test_gemm_f16_zero_weighted_outlier_at_the_limit(M, K, N):
    w, x, k0 = zero_column_case(3, M, K, N)
    limit = 2.0 ** C_GEMM_F16 * ratio_min(w, M, K, x, None)
    wd = dev(w)
    for big in (1e4, 1e6, 2.0 ** 24, 0.9 * limit, -0.9 * limit):
        if abs(big) > limit:
            continue
        xb = with_outlier(x, k0, big)
        y = run_mul_mat(wd, M, K, xb, B.Q2_0_PREC_F16_MFMA)
        assert_products(y, w, M, K, xb, REL_F16,
                        what="fp16 GEMM M=%d K=%d N=%d outlier %.4g (limit %.4g)" % (M, K, N, big, limit))


# ------------------------------------------------------------------ Q2_0_PREC_F32: no range condition

@pytest.mark.parametrize("M,K,N", [(300, 4096, 1), (16400, 4096, 2), (300, 2048, 8), (200, 4096, 40)])
def test_prec_f32_has_no_range_condition(M, K, N):
    w, x, k0 = zero_column_case(4, M, K, N)
    rows = rows_of(M)
    wd = dev(w)
    for big in (1e6, 2.0 ** 24, 1e15, 1e30, -1e30):
        xb = with_outlier(x, k0, big)
        y = run_mul_mat(wd, M, K, xb, B.Q2_0_PREC_F32)
        assert_products(y, w, M, K, xb, REL_F32, rows=rows,
                        what="PREC_F32 M=%d K=%d N=%d outlier %.3g" % (M, K, N, big))


def test_prec_f32_small_n_is_the_generic_kernel():
    """PREC_F32 with N <= 8 runs the f32 generic kernel: bit for bit what the mat-vec gives
    when the weights sit at a 2-byte offset (which only that kernel takes)."""
    torch = __import__("torch")
    M, K = 300, 1024
    w = synth.weight(13, 0, 0, M, K, "quad", synth.ScaleDist("uniform", 0.01, 0.1))
    wd = dev(w)
    raw = torch.zeros(w.size + 2, dtype=torch.uint8, device="cuda")
    raw[2:] = wd.view(-1)
    w_off = raw[2:]
    for N in (1, 5, 8):
        x = synth.activations(13, 0, N, N, K)
        a = run_mat_vec(w_off, M, K, x)
        assert np.array_equal(run_mul_mat(wd, M, K, x, B.Q2_0_PREC_F32).view(np.uint32), a.view(np.uint32))


def test_mul_mat_id_prec_f32_few_tokens_has_no_range_condition():
    torch = __import__("torch")
    E, M, K, U, T = 6, 200, 1024, 2, 3
    k0 = 64 * K0_BLOCK + K0_OFF
    experts = []
    for e in range(E):
        w, _, _ = zero_column_case(10 + e, M, K, 1)
        experts.append(w)
    wall = np.concatenate(experts, axis=0)
    x = synth.activations(50, 0, 0, T, K)
    x[:, k0] = 1e30
    ids = np.array([[0, 5], [3, 3], [1, 2]], dtype=np.int32)
    y = B.q2_0_mul_mat_id(dev(wall), E, M, K, dev(x), dev(ids), precision=B.Q2_0_PREC_F32)
    y = y.cpu().numpy()
    for t in range(T):
        for u in range(U):
            e = int(ids[t, u])
            assert_products(y[t * U + u][None, :], experts[e], M, K, x[t][None, :], REL_F32,
                            what="expert %d token %d" % (e, t))


# ------------------------------------------------------------------ Qwen3-8B prefill shapes

def planned_splits(M, K, N):
    """The K split q2_0_mul_mat plans, read from its workspace size (x16 + exponents +
    splits * N * M partial floats)."""
    need = B.mul_mat_workspace_bytes(M, K, N, B.Q2_0_PREC_F16_MFMA)
    base = -(-N * K * 2 // 256) * 256 + -(-N * 4 // 256) * 256
    return 1 if need == base else (need - base) // (N * M * 4)


def test_mul_mat_8b_o_two_way_split():
    wl = synth.STACK_8B
    M, K = wl.shapes["o"]
    N = 512
    assert planned_splits(M, K, N) == 2, "the 8B o projection at N = 512 is planned as a 2-way K split"
    w = ws(wl, "o", layer=2)
    x = synth.activations(wl.seed, 2, synth.stack_x_matrix_index(K) + 21, N, K)
    y = run_mul_mat(dev(w), M, K, x, B.Q2_0_PREC_F16_MFMA)
    rows = np.unique(np.concatenate([np.arange(0, M, 37), np.arange(M - 24, M)]))
    assert_products(y, w, M, K, x, REL_F16, rows=rows, what="8B o, 2-way split")


def test_mul_mat_group_8b_qkv():
    wl = synth.STACK_8B
    names = ["q", "k", "v"]
    K = wl.shapes["q"][1]
    mats = [(ws(wl, n, layer=5), wl.shapes[n][0]) for n in names]
    x = synth.activations(wl.seed, 5, synth.stack_x_matrix_index(K) + 22, 512, K)
    ys = run_gemm_group(mats, K, x, B.Q2_0_PREC_F16_MFMA)
    for (w, M), y, n in zip(mats, ys, names):
        rows = np.unique(np.concatenate([np.arange(0, M, 53), np.arange(M - 16, M)]))
        assert_products(y, w, M, K, x, REL_F16, rows=rows, what="8B q/k/v group: " + n)
