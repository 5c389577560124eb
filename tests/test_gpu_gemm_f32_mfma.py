"""Q2_0_PREC_F32_MFMA, the fp32-grade GEMM on the matrix cores, against the fp64 oracle.

Its contract (include/q2_0.h): |y - y_exact| <= 1e-5 * A for finite x with |x| < 2^100,
|d| <= 32752 and K <= 16384 under the mat-vec's range condition
    max_k |x[n][k]| * sum_k |W[m][k]| <= 2^21 * A[n][m],   A = sum_k |W[m][k] x[n][k]|.
The ordinary parity cases (ragged shapes, the 1.7B prefill and 8B stack shapes, groups,
activation ranges, all-zero weights, scaling) run in test_gpu_parity.py with the other
precisions; here are the cases particular to this path:
  * a large activation that meets only zero weights, at 0.9 of the range limit;
  * scales at the limit |d| = 32752, where d*(q-1) still fits fp16;
  * the K splits the planner takes (their partials are summed in a fixed order) and
    deterministic results;
  * weights at a 2-byte offset (the 2-byte code loads), bit for bit the aligned result;
  * N <= 8, which is the mat-vec bit for bit; 16-bit activations, bit for bit the f32
    call with the same values; q2_0_mul_mat_noalloc; q2_0_mul_mat_id (which runs this
    precision as Q2_0_PREC_F32).
"""

import numpy as np
import pytest

import oracle
from ternary_bit_quantized_amd import q2_0 as B
from ternary_bit_quantized_amd import synth
from test_gpu_accuracy import ratio_min, rows_of, with_outlier, zero_column_case
from test_gpu_parity import REL_F32, assert_products, dev, host, run_gemm_group, run_mat_vec, run_mul_mat, ws

pytestmark = pytest.mark.gpu

P = B.Q2_0_PREC_F32_MFMA
C_RANGE = 21


def bits_equal(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


def planned_splits(M, K, N):
    """The K split of a single-matrix call, read from its workspace size (x as two fp16
    halves + exponents + splits * N * M partial floats)."""
    need = B.mul_mat_workspace_bytes(M, K, N, P)
    base = -(-N * K * 4 // 256) * 256 + -(-N * 4 // 256) * 256
    return 1 if need == base else (need - base) // (N * M * 4)


@pytest.mark.parametrize("M,K,N", [(1024, 4096, 64), (256, 12288, 16), (300, 2048, 130), (129, 16384, 40)])
def test_zero_weighted_outlier_at_the_limit(M, K, N):
    w, x, k0 = zero_column_case(5, M, K, N)
    limit = 2.0 ** C_RANGE * ratio_min(w, M, K, x, None)
    wd = dev(w)
    for big in (1e4, 1e6, 0.9 * limit, -0.9 * limit):
        if abs(big) > limit:
            continue
        xb = with_outlier(x, k0, big)
        y = run_mul_mat(wd, M, K, xb, P)
        assert_products(y, w, M, K, xb, REL_F32,
                        what="F32_MFMA M=%d K=%d N=%d outlier %.4g (limit %.4g)" % (M, K, N, big, limit))


def test_scales_at_the_fp16_limit():
    """|d| = 32752 (d*(q-1) = -32752 .. 65504, still finite fp16) and d = 0 blocks."""
    rng = np.random.default_rng(61)
    M, K, N = 200, 1024, 24
    codes = rng.integers(0, 4, size=(M, K), dtype=np.uint8)
    d = rng.choice(np.array([32752.0, -32752.0, 0.0, 1.0], dtype=np.float16), size=(M, K // 64))
    w = synth.pack(codes, d)
    x = rng.standard_normal((N, K)).astype(np.float32)
    y = run_mul_mat(dev(w), M, K, x, P)
    assert_products(y, w, M, K, x, REL_F32, what="|d| = 32752")


@pytest.mark.parametrize("M,K,N", [(120, 1536, 60), (256, 12288, 16), (4096, 4096, 512)])
def test_k_splits_and_determinism(M, K, N):
    """Calls whose tile grid is too small for the GPU take a K split; each split's partial
    is rounded to f32 once and the partials are added in split order, so results repeat
    bit for bit."""
    sp = planned_splits(M, K, N)
    w = synth.weight(62, M, N, M, K, "quad", synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.02))
    x = synth.activations(62, M, N, N, K)
    wd = dev(w)
    a = run_mul_mat(wd, M, K, x, P)
    b = run_mul_mat(wd, M, K, x, P)
    assert bits_equal(a, b), "run-to-run difference (split %d)" % sp
    rows = rows_of(M)
    assert_products(a, w, M, K, x, REL_F32, rows=rows, what="M=%d K=%d N=%d split %d" % (M, K, N, sp))


def test_split_planned_somewhere():
    """The cases above include at least one K split (the planner's choice is a model, so
    this pins that the split path is exercised, not its exact count)."""
    assert max(planned_splits(M, K, N) for M, K, N in [(120, 1536, 60), (256, 12288, 16), (4096, 4096, 512)]) > 1


def test_wide_n_many_column_tiles():
    """N = 1500: 24 column tiles of 64 (no XCD column map), a ragged last one, sampled
    rows and every column against the oracle."""
    M, K, N = 260, 2048, 1500
    w = synth.weight(68, M, N, M, K, "quad", synth.ScaleDist("uniform", 0.005, 0.05))
    x = synth.activations(68, M, N, N, K)
    y = run_mul_mat(dev(w), M, K, x, P)
    rows = np.unique(np.concatenate([np.arange(0, M, 17), [M - 1]]))
    assert_products(y, w, M, K, x, REL_F32, rows=rows, what="N=%d" % N)


def test_weights_at_two_byte_offset():
    torch = __import__("torch")
    for M, K, N in [(200, 512, 130), (333, 640, 70)]:
        w = synth.weight(63, M, N, M, K, "quad", synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.02))
        flat = np.ascontiguousarray(w).reshape(-1)
        buf = torch.zeros(flat.size + 16, dtype=torch.uint8, device="cuda")
        buf[2:2 + flat.size].copy_(torch.from_numpy(flat).cuda())
        w_off = buf[2:]
        assert w_off.data_ptr() % 4 == 2
        x = synth.activations(63, M, N, N, K)
        y_al = run_mul_mat(dev(w), M, K, x, P)
        y_off = run_mul_mat(w_off, M, K, x, P)
        assert bits_equal(y_al, y_off), "M=%d: offset W changed the result" % M
        assert_products(y_off, w, M, K, x, REL_F32, what="offset W M=%d K=%d" % (M, K))


def test_small_n_is_the_mat_vec():
    M, K = 300, 1024
    w = synth.weight(64, 0, 0, M, K, "quad", synth.ScaleDist("uniform", 0.01, 0.1))
    wd = dev(w)
    for N in (1, 2, 5, 8):
        x = synth.activations(64, 0, N, N, K)
        assert bits_equal(run_mul_mat(wd, M, K, x, P), run_mat_vec(wd, M, K, x))


def test_f16_and_bf16_activations_match_f32():
    """Activations given as fp16 or bf16 are converted exactly to f32 first: the results
    are bit for bit those of the f32 call on the same values."""
    torch = __import__("torch")
    M, K, N = 260, 2048, 33
    w = synth.weight(65, M, N, M, K, "quad", synth.ScaleDist("uniform", 0.005, 0.05))
    wd = dev(w)
    x32 = synth.activations(65, M, N, N, K)
    for dt, xt in ((torch.float16, B.Q2_0_ACT_F16), (torch.bfloat16, B.Q2_0_ACT_BF16)):
        xh = torch.from_numpy(x32).to(dt).cuda()
        xf = xh.float().cpu().numpy()
        ref = run_mul_mat(wd, M, K, xf, P)
        y = torch.full((N, M), float("nan"), dtype=torch.float32, device="cuda")
        need = B.mul_mat_workspace_bytes(M, K, N, P)
        wsd = torch.empty(need, dtype=torch.uint8, device="cuda")
        st = B.mul_mat_act_raw(wd.data_ptr(), M, K, xh.data_ptr(), xt, K, N, y.data_ptr(), M, P, wsd.data_ptr(),
                               need, torch.cuda.current_stream().cuda_stream)
        assert st == 0, B.lib().q2_0_status_string(st)
        assert bits_equal(host(y), ref), str(dt)


def test_noalloc_matches_workspace_call():
    torch = __import__("torch")
    M, K, N = 700, 4096, 100
    w = synth.weight(66, M, N, M, K, "quad", synth.ScaleDist("uniform", 0.005, 0.05))
    wd = dev(w)
    x = synth.activations(66, M, N, N, K)
    ref = run_mul_mat(wd, M, K, x, P)
    xd = dev(x)
    y = torch.full((N, M), float("nan"), dtype=torch.float32, device="cuda")
    st = B.mul_mat_noalloc_raw(wd.data_ptr(), M, K, xd.data_ptr(), K, N, y.data_ptr(), M, P,
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().q2_0_status_string(st)
    assert bits_equal(host(y), ref)


def test_group_8b_qkv():
    wl = synth.STACK_8B
    names = ["q", "k", "v"]
    K = wl.shapes["q"][1]
    mats = [(ws(wl, n, layer=7), wl.shapes[n][0]) for n in names]
    x = synth.activations(wl.seed, 7, synth.stack_x_matrix_index(K) + 23, 512, K)
    ys = run_gemm_group(mats, K, x, P)
    for (w, M), y, n in zip(mats, ys, names):
        rows = np.unique(np.concatenate([np.arange(0, M, 71), np.arange(M - 16, M)]))
        assert_products(y, w, M, K, x, REL_F32, rows=rows, what="8B q/k/v group, F32_MFMA: " + n)


def test_mul_mat_id_runs_as_prec_f32():
    E, M, K, U, T = 6, 200, 1024, 2, 12
    wall = synth.weight(67, 0, 0, E * M, K, "quad", synth.ScaleDist("uniform", 0.005, 0.05))
    x = synth.activations(67, 0, 1, T, K)
    rng = np.random.default_rng(67)
    ids = rng.integers(0, E, size=(T, U)).astype(np.int32)
    wd, xd, idd = dev(wall), dev(x), dev(ids)
    a = B.q2_0_mul_mat_id(wd, E, M, K, xd, idd, precision=P).cpu().numpy()
    b = B.q2_0_mul_mat_id(wd, E, M, K, xd, idd, precision=B.Q2_0_PREC_F32).cpu().numpy()
    assert bits_equal(a, b)
    e = int(ids[3, 1])
    y_ref, bound = oracle.mul_mat(wall[e * M:(e + 1) * M], M, K, x[3][None, :])
    r = oracle.check_products(a[3 * U + 1][None, :], y_ref, bound, REL_F32)
    assert r["ok"], r
