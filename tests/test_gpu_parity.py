"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

get_rows must match bit for bit (NaN matches NaN).  Products must satisfy
|y - y_ref| <= rel * sum|W x| elementwise with rel = 1e-5 on the fp32 paths (mat-vec
and the fp32 GEMM) and 2e-3 on the fp16-MFMA GEMM; a non-finite y fails where y_ref is
finite, and a zero bound demands y == 0 exactly.  Large workloads run at full size on
the GPU and are compared on sampled rows the oracle computes one by one.
"""

import numpy as np
import pytest

import oracle
from ternary_bit_quantized_amd import q2_0 as B
from ternary_bit_quantized_amd import synth

pytestmark = pytest.mark.gpu

REL_F32 = 1e-5
REL_F16 = 2e-3


def _torch():
    import torch
    return torch


def dev(a):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    _torch().cuda.synchronize()
    return t.cpu().numpy()


def same_bits(a, b):
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    nan = np.isnan(a) & np.isnan(b)
    eq = nan | (a.view(np.uint32) == b.view(np.uint32))
    return bool(eq.all()), int((~eq).sum())


def assert_products(y, w, M, K, x, rel, rows=None, what=""):
    y_ref, bound = oracle.mul_mat(w, M, K, x, rows=rows)
    yy = y if rows is None else y[:, rows]
    r = oracle.check_products(yy, y_ref, bound, rel)
    assert r["ok"], "%s: %d/%d outside %.0e*bound, worst %.3g, first %s" % (
        what, r["n_bad"], r["n"], rel, r["max_err_over_bound"], r["first_bad"])
    return r


def run_mat_vec(w_d, M, K, x, ldx=None, ldy=None):
    torch = _torch()
    N = x.shape[0]
    ldx = ldx or K
    ldy = ldy or M
    xb = np.zeros((N, ldx), dtype=np.float32)
    xb[:, :K] = x
    xd = dev(xb)
    yd = torch.full((N, ldy), float("nan"), dtype=torch.float32, device="cuda")
    st = B.mul_mat_vec_raw(w_d.data_ptr(), M, K, xd.data_ptr(), ldx, N, yd.data_ptr(), ldy,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().q2_0_status_string(st)
    y = host(yd)
    if ldy > M:
        assert np.all(np.isnan(y[:, M:])), "mat-vec wrote past M"
    return y[:, :M]


def run_mul_mat(w_d, M, K, x, precision, ldx=None, ldy=None):
    torch = _torch()
    N = x.shape[0]
    ldx = ldx or K
    ldy = ldy or M
    xb = np.zeros((N, ldx), dtype=np.float32)
    xb[:, :K] = x
    xd = dev(xb)
    yd = torch.full((N, ldy), float("nan"), dtype=torch.float32, device="cuda")
    ws = B.mul_mat_workspace_bytes(M, K, N, precision)
    wsd = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
    st = B.mul_mat_raw(w_d.data_ptr(), M, K, xd.data_ptr(), ldx, N, yd.data_ptr(), ldy, precision,
                       wsd.data_ptr(), ws, torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().q2_0_status_string(st)
    y = host(yd)
    if ldy > M:
        assert np.all(np.isnan(y[:, M:])), "mul_mat wrote past M"
    return y[:, :M]


def run_get_rows(w_d, M, K, ids, ld_out=None, offset=0):
    torch = _torch()
    ld = ld_out or K
    n = ids.size
    buf = torch.full((n * ld + offset + 16,), float("nan"), dtype=torch.float32, device="cuda")
    sentinel = np.float32(-12345.5)
    buf.fill_(float(sentinel))
    idd = dev(ids.astype(np.int32))
    st = B.get_rows_raw(w_d.data_ptr(), M, K, idd.data_ptr(), n, buf.data_ptr() + 4 * offset, ld,
                        torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().q2_0_status_string(st)
    flat = host(buf)
    assert np.all(flat[:offset] == sentinel) and np.all(flat[offset + n * ld:] == sentinel)
    out = flat[offset:offset + n * ld].reshape(n, ld)
    if ld > K:
        assert np.all(out[:, K:] == sentinel), "get_rows wrote past K"
    return out[:, :K]


def ws(wl, name="w", layer=0):
    return synth.workload_weight(wl, name, layer)


# =============================================================================== get_rows

def test_get_rows_tiny_workload():
    M, K = synth.TINY.shapes["w"]
    w = ws(synth.TINY)
    ids = synth.row_ids(synth.TINY.seed, 0, 0, synth.TINY_IDS, M)
    out = run_get_rows(dev(w), M, K, ids)
    ok, nbad = same_bits(out, oracle.get_rows(w, M, K, ids))
    assert ok, nbad


def test_get_rows_every_half_scale():
    rng = np.random.default_rng(0)
    M, K = 65536, 64
    w = synth.random_blocks(rng, M, 1)
    w[:, 0] = (np.arange(M) & 0xFF).astype(np.uint8)
    w[:, 1] = (np.arange(M) >> 8).astype(np.uint8)
    ids = np.arange(M, dtype=np.int32)
    out = run_get_rows(dev(w), M, K, ids)
    ok, nbad = same_bits(out, oracle.get_rows(w, M, K, ids))
    assert ok, nbad


@pytest.mark.parametrize("M,K,n,ld,off", [(300, 192, 14000, 192, 0), (77, 64, 500, 70, 1),
                                          (1000, 4096, 64, 4100, 3), (5, 128, 33, 128, 2)])
def test_get_rows_random_bytes_fuzz(M, K, n, ld, off):
    rng = np.random.default_rng(M + K + n)
    w = synth.random_blocks(rng, M, K // 64)
    ids = rng.integers(-3, M + 3, size=n).astype(np.int32)
    ids[:4] = [0, M - 1, -1, M]
    out = run_get_rows(dev(w), M, K, ids, ld_out=ld, offset=off)
    ok, nbad = same_bits(out, oracle.get_rows(w, M, K, ids))
    assert ok, nbad
    assert np.all(np.isnan(out[(ids < 0) | (ids >= M)]))


def test_get_rows_vocab_workload():
    wl = synth.VOCAB_8B
    M, K = wl.shapes["emb"]
    w = ws(wl, "emb")
    ids = synth.row_ids(wl.seed, 0, 0, synth.VOCAB_IDS, M)
    out = run_get_rows(dev(w), M, K, ids)
    ok, nbad = same_bits(out, oracle.get_rows(w, M, K, ids))
    assert ok, nbad


# =============================================================================== mat-vec

@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7, 8])
def test_mat_vec_tiny_all_n(N):
    M, K = synth.TINY.shapes["w"]
    w = ws(synth.TINY)
    x = synth.activations(synth.TINY.seed, 0, 0, N, K)
    y = run_mat_vec(dev(w), M, K, x)
    assert_products(y, w, M, K, x, REL_F32, what="tiny N=%d" % N)


@pytest.mark.parametrize("M,K,N,ldx,ldy,codes", [
    (1, 64, 1, 64, 1, "quad"), (257, 192, 3, 200, 300, "quad"), (63, 576, 8, 577, 64, "tern"),
    (129, 4096, 2, 4096, 129, "quad"), (31, 12288, 5, 12288, 40, "tern_c3"), (1000, 64 * 9, 1, 577, 1000, "quad"),
    (4095, 2048, 8, 2048, 4095, "quad"), (16, 512 + 64, 4, 600, 16, "quad")])
def test_mat_vec_ragged_and_strided(M, K, N, ldx, ldy, codes):
    w = synth.weight(11, M, K // 64, M, K, codes, synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.02))
    x = synth.activations(11, M, K // 64, N, K)
    y = run_mat_vec(dev(w), M, K, x, ldx=ldx, ldy=ldy)
    assert_products(y, w, M, K, x, REL_F32, what="M=%d K=%d N=%d" % (M, K, N))


@pytest.mark.parametrize("code,factor", [(1, 0.0), (2, 1.0), (0, -1.0), (3, 2.0)])
def test_mat_vec_closed_forms(code, factor):
    rng = np.random.default_rng(code)
    M, K, N = 96, 2048, 4
    d = rng.uniform(0.001, 0.1, size=(M, K // 64)).astype(np.float16)
    codes = np.full((M, K), code, dtype=np.uint8)
    w = synth.pack(codes, d)
    x = rng.standard_normal((N, K), dtype=np.float32)
    y = run_mat_vec(dev(w), M, K, x)
    if factor == 0.0:
        assert np.all(y == 0.0)
    expect = factor * (x.astype(np.float64).reshape(N, K // 64, 64).sum(-1) @ d.astype(np.float64).T)
    _, bound = oracle.mul_mat(w, M, K, x)
    assert np.all(np.abs(y - expect) <= REL_F32 * bound)


def test_mat_vec_decode_1p7b_workload():
    wl = synth.DECODE_1P7B
    for name, (M, K) in wl.shapes.items():
        w = ws(wl, name)
        wd = dev(w)
        for N in wl.ns:
            x = synth.activations(wl.seed, 0, synth.MATS.index(name), N, K)
            y = run_mat_vec(wd, M, K, x)
            assert_products(y, w, M, K, x, REL_F32, what="%s N=%d" % (name, N))


def test_mat_vec_stack_8b_layer_workload():
    wl = synth.STACK_8B
    rng = np.random.default_rng(3)
    for name, (M, K) in wl.shapes.items():
        w = ws(wl, name, layer=35)
        x = synth.activations(wl.seed, 0, synth.stack_x_matrix_index(K), 1, K)
        y = run_mat_vec(dev(w), M, K, x)
        rows = np.unique(np.concatenate([rng.integers(0, M, 512), [0, M - 1]]))
        assert_products(y, w, M, K, x, REL_F32, rows=rows, what=name)


@pytest.mark.parametrize("N", [1, 4])
def test_mat_vec_vocab_head_workload(N):
    wl = synth.VOCAB_8B
    M, K = wl.shapes["emb"]
    w = ws(wl, "emb")
    x = synth.activations(wl.seed, 0, 0, N, K)
    y = run_mat_vec(dev(w), M, K, x)
    rows = np.unique(np.concatenate([np.random.default_rng(N).integers(0, M, 2048), [0, M - 1]]))
    assert_products(y, w, M, K, x, REL_F32, rows=rows, what="head N=%d" % N)


def test_mat_vec_metamorphic_scale_and_permute():
    rng = np.random.default_rng(21)
    M, K, N = 200, 1024, 3
    codes = rng.integers(0, 4, size=(M, K), dtype=np.uint8)
    d = rng.uniform(0.01, 0.1, size=(M, K // 64)).astype(np.float16)
    x = rng.standard_normal((N, K), dtype=np.float32)
    y = run_mat_vec(dev(synth.pack(codes, d)), M, K, x)
    y4 = run_mat_vec(dev(synth.pack(codes, (d.astype(np.float32) * 4).astype(np.float16))), M, K, x)
    assert np.array_equal(y4, 4 * y)
    perm = rng.permutation(M)
    yp = run_mat_vec(dev(synth.pack(codes[perm], d[perm])), M, K, x)
    assert np.array_equal(yp, y[:, perm])
    for n in range(N):
        y1 = run_mat_vec(dev(synth.pack(codes, d)), M, K, x[n:n + 1])
        _, bound = oracle.mul_mat(synth.pack(codes, d), M, K, x[n:n + 1])
        assert np.all(np.abs(y1[0] - y[n]) <= 2 * REL_F32 * bound[0])


# Activation magnitudes far from 1: fp16 staging must neither overflow (|x| > 65504)
# nor lose the small end to fp16 subnormals, so each column is scaled into range.
MAGS = [1e-30, 1e-8, 1e-5, 1e-3, 1.0, 3e3, 1e5, 1e8, 1e30]


def _ranged_x(seed, N, K, mags, spread=False):
    x = synth.activations(seed, 0, 9, N, K).astype(np.float64)
    x *= np.array([mags[n % len(mags)] for n in range(N)])[:, None]
    if spread:   # every other element 1e4 times smaller: dynamic range inside a column
        x[:, 1::2] *= 1e-4
    return x.astype(np.float32)


# K-split kernel; streaming kernel with a ragged half stage (K = 512) and with whole stages
@pytest.mark.parametrize("M,K", [(300, 1024), (16400, 512), (16400, 4096)])
@pytest.mark.parametrize("N,first", [(1, 0), (1, 2), (1, 7), (1, 8), (4, 0), (8, 1)])
def test_mat_vec_activation_range(M, K, N, first):
    w = synth.weight(13, M, K // 64, M, K, "tern_c3", synth.ScaleDist("uniform", 0.005, 0.05))
    mags = MAGS[first:] + MAGS[:first]
    for spread in (False, True):
        x = _ranged_x(13, N, K, mags, spread)
        y = run_mat_vec(dev(w), M, K, x)
        rows = None if M < 1000 else np.arange(0, M, 7)
        assert_products(y, w, M, K, x, REL_F32, rows=rows,
                        what="M=%d N=%d mags from %g spread=%s" % (M, N, mags[0], spread))


# K-split kernel; streaming kernel with a ragged half stage (K = 512) and with whole stages
@pytest.mark.parametrize("M,K", [(300, 1024), (16400, 512), (16400, 4096)])
@pytest.mark.parametrize("big", [1e4, 1e6])
def test_mat_vec_outlier_on_zero_weights(M, K, big):
    """A huge activation whose weights are all zero must not cost the other elements
    their accuracy: the bound is relative to sum|W x|, which the outlier does not enter."""
    rng = synth.rng_for(16, M, K, 0)
    codes = rng.integers(0, 3, size=(M, K), dtype=np.uint8)
    k0 = 3 * 64 + 17
    codes[:, k0] = 1
    d = rng.uniform(0.005, 0.05, size=(M, K // 64)).astype(np.float16)
    w = synth.pack(codes, d)
    x = synth.activations(16, M, K, 2, K)
    x[:, k0] = big
    x[1, k0 + 5] = -big * 0.5   # a second outlier with live weights in the same block
    y = run_mat_vec(dev(w), M, K, x)
    rows = None if M < 1000 else np.arange(0, M, 7)
    assert_products(y, w, M, K, x, REL_F32, rows=rows, what="outlier %g M=%d" % (big, M))


def test_mat_vec_group_activation_range():
    K, N = 512, 3
    mats = [synth.weight(14, i, 0, M, K, "quad", synth.ScaleDist("uniform", 0.005, 0.05))
            for i, M in enumerate((16384, 80, 4096))]
    x = _ranged_x(14, N, K, [1e-9, 7e4, 1e12])
    ys = run_group([(w, w.shape[0]) for w in mats], K, x)
    for w, y in zip(mats, ys):
        M = w.shape[0]
        assert_products(y, w, M, K, x, REL_F32, rows=np.arange(0, M, 5), what="group M=%d" % M)


# =============================================================================== GEMM

@pytest.mark.parametrize("precision,rel", [(B.Q2_0_PREC_F16_MFMA, REL_F16), (B.Q2_0_PREC_F32, REL_F32),
                                             (B.Q2_0_PREC_F32_MFMA, REL_F32)])
@pytest.mark.parametrize("M,K,N,ldx,ldy", [
    (64, 64, 64, 64, 64), (1, 64, 9, 64, 1), (65, 192, 63, 200, 70), (200, 512, 130, 512, 203),
    (127, 2048, 65, 2050, 127), (33, 576, 100, 576, 33),
    # one tile: K split 3 ways (24 blocks) and 6 ways (48 blocks), ragged rows and columns
    (120, 1536, 60, 1536, 121), (127, 3072, 63, 3080, 127)])
def test_mul_mat_ragged(precision, rel, M, K, N, ldx, ldy):
    w = synth.weight(12, M, N, M, K, "quad", synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.02))
    x = synth.activations(12, M, N, N, K)
    y = run_mul_mat(dev(w), M, K, x, precision, ldx=ldx, ldy=ldy)
    assert_products(y, w, M, K, x, rel, what="p=%d M=%d K=%d N=%d" % (precision, M, K, N))


@pytest.mark.parametrize("precision,rel", [(B.Q2_0_PREC_F16_MFMA, REL_F16), (B.Q2_0_PREC_F32, REL_F32),
                                             (B.Q2_0_PREC_F32_MFMA, REL_F32)])
def test_mul_mat_prefill_1p7b_workload(precision, rel):
    wl = synth.PREFILL_1P7B
    rng = np.random.default_rng(2)
    for name, (M, K) in wl.shapes.items():
        w = ws(wl, name)
        x = synth.activations(wl.seed, 0, synth.MATS.index(name), 512, K)
        y = run_mul_mat(dev(w), M, K, x, precision)
        rows = np.unique(np.concatenate([rng.integers(0, M, 96), [0, M - 1]]))
        assert_products(y, w, M, K, x, rel, rows=rows, what=name)


@pytest.mark.parametrize("precision,rel", [(B.Q2_0_PREC_F16_MFMA, REL_F16), (B.Q2_0_PREC_F32, REL_F32),
                                             (B.Q2_0_PREC_F32_MFMA, REL_F32)])
def test_mul_mat_stack_8b_workload(precision, rel):
    wl = synth.STACK_8B
    rng = np.random.default_rng(4)
    for name in ("k", "down"):
        M, K = wl.shapes[name]
        w = ws(wl, name, layer=0)
        x = synth.activations(wl.seed, 0, synth.stack_x_matrix_index(K) + 10, 512, K)
        y = run_mul_mat(dev(w), M, K, x, precision)
        rows = np.unique(np.concatenate([rng.integers(0, M, 48), [0, M - 1]]))
        assert_products(y, w, M, K, x, rel, rows=rows, what=name)


def test_weights_at_two_byte_offset():
    """W at an address 2 mod 4 (the API's minimum alignment for 18-byte blocks): the GEMM
    then reads its codes with 2-byte loads, in both tile configurations (200 x 512 at
    N = 130: 128-row tiles; 65357 x 640 at N = 500: 256-row tiles).  The results are bit
    for bit those of the same W at an aligned address, and within the fp16 bound of the
    oracle; get_rows and the mat-vec are checked on the offset W too."""
    torch = _torch()
    for M, K, N in [(200, 512, 130), (65357, 640, 500)]:
        w = synth.weight(31, M, N, M, K, "quad", synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.02))
        flat = np.ascontiguousarray(w).reshape(-1)
        buf = torch.zeros(flat.size + 16, dtype=torch.uint8, device="cuda")
        buf[2:2 + flat.size].copy_(torch.from_numpy(flat).cuda())
        w_off = buf[2:]
        assert w_off.data_ptr() % 4 == 2
        x = synth.activations(31, M, N, N, K)
        y_al = run_mul_mat(dev(w), M, K, x, B.Q2_0_PREC_F16_MFMA)
        y_off = run_mul_mat(w_off, M, K, x, B.Q2_0_PREC_F16_MFMA)
        assert np.array_equal(y_al.view(np.uint32), y_off.view(np.uint32)), "M=%d: offset W changed the GEMM" % M
        rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 200)), [M - 1]]))
        assert_products(y_off, w, M, K, x, REL_F16, rows=rows, what="offset W M=%d" % M)
        x1 = x[:1]
        y1 = run_mat_vec(w_off, M, K, x1)
        assert_products(y1, w, M, K, x1, REL_F32, rows=rows, what="offset W mat-vec M=%d" % M)
        ids = np.array([0, M - 1, M // 2, 7 % M], dtype=np.int32)
        out = run_get_rows(w_off, M, K, ids)
        ok, nbad = same_bits(out, oracle.get_rows(w, M, K, ids))
        assert ok, "offset W get_rows M=%d: %d values differ" % (M, nbad)


def test_mul_mat_small_n_routes_to_mat_vec():
    """The fast precision with N <= 8 is the mat-vec, bit for bit; the fp32 precision is
    the f32 generic kernel (bitwise checks of that in test_gpu_accuracy.py)."""
    M, K = 300, 1024
    w = synth.weight(13, 0, 0, M, K, "quad", synth.ScaleDist("uniform", 0.01, 0.1))
    wd = dev(w)
    for N in (1, 5, 8):
        x = synth.activations(13, 0, N, N, K)
        a = run_mat_vec(wd, M, K, x)
        assert np.array_equal(run_mul_mat(wd, M, K, x, B.Q2_0_PREC_F16_MFMA), a)
        assert_products(run_mul_mat(wd, M, K, x, B.Q2_0_PREC_F32), w, M, K, x, REL_F32, what="PREC_F32 N=%d" % N)


@pytest.mark.parametrize("precision,rel", [(B.Q2_0_PREC_F16_MFMA, REL_F16), (B.Q2_0_PREC_F32, REL_F32),
                                             (B.Q2_0_PREC_F32_MFMA, REL_F32)])
@pytest.mark.parametrize("M,K,N", [(200, 640, 9), (1024, 4096, 27), (129, 12288, 18)])
def test_mul_mat_activation_range(precision, rel, M, K, N):
    w = synth.weight(15, M, K // 64, M, K, "tern", synth.ScaleDist("uniform", 0.002, 0.02))
    for spread in (False, True):
        x = _ranged_x(15, N, K, MAGS, spread)
        y = run_mul_mat(dev(w), M, K, x, precision)
        assert_products(y, w, M, K, x, rel, what="M=%d K=%d N=%d spread=%s" % (M, K, N, spread))


@pytest.mark.parametrize("precision", [B.Q2_0_PREC_F16_MFMA, B.Q2_0_PREC_F32, B.Q2_0_PREC_F32_MFMA])
def test_mul_mat_all_code_one_is_exactly_zero(precision):
    rng = np.random.default_rng(5)
    M, K, N = 130, 1024, 70
    d = rng.uniform(0.01, 1.0, size=(M, K // 64)).astype(np.float16)
    w = synth.pack(np.ones((M, K), dtype=np.uint8), d)
    x = rng.standard_normal((N, K), dtype=np.float32)
    y = run_mul_mat(dev(w), M, K, x, precision)
    assert np.all(y == 0.0)


@pytest.mark.parametrize("precision", [B.Q2_0_PREC_F16_MFMA, B.Q2_0_PREC_F32, B.Q2_0_PREC_F32_MFMA])
def test_mul_mat_metamorphic_scale(precision):
    rng = np.random.default_rng(6)
    M, K, N = 100, 512, 40
    codes = rng.integers(0, 4, size=(M, K), dtype=np.uint8)
    d = rng.uniform(0.01, 0.1, size=(M, K // 64)).astype(np.float16)
    x = rng.standard_normal((N, K), dtype=np.float32)
    y = run_mul_mat(dev(synth.pack(codes, d)), M, K, x, precision)
    y8 = run_mul_mat(dev(synth.pack(codes, (d.astype(np.float32) * 8).astype(np.float16))), M, K, x,
                     precision)
    assert np.array_equal(y8, 8 * y)


# =============================================================================== grouped mat-vec

def run_group(mats, K, x, ldx=None):
    """mats: [(w_bytes or None, M, codes)]; runs q2_0_mul_mat_vec_group, returns [y_i]."""
    torch = _torch()
    N = x.shape[0]
    ldx = ldx or K
    xb = np.zeros((N, ldx), dtype=np.float32)
    xb[:, :K] = x
    xd = dev(xb)
    keep, entries, ys = [], [], []
    for w, M in mats:
        wd = dev(w) if M else None
        yd = torch.full((N, M + 3), float("nan"), dtype=torch.float32, device="cuda")
        keep.append(wd)
        ys.append(yd)
        entries.append((wd.data_ptr() if wd is not None else 0, M, yd.data_ptr(), M + 3))
    items = B.make_items(entries)
    st = B.mul_mat_vec_group_raw(items, len(entries), K, xd.data_ptr(), ldx, N,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().q2_0_status_string(st)
    out = []
    for (w, M), yd in zip(mats, ys):
        y = host(yd)
        assert np.all(np.isnan(y[:, M:])), "group wrote past M"
        out.append(y[:, :M])
    return out


@pytest.mark.parametrize("N", [1, 2, 5, 8])
def test_mat_vec_group_qkv_like(N):
    K = 2048
    shapes = [4096, 1024, 1024, 0, 37, 16, 1]
    mats = [(synth.weight(20, i, N, M, K, "quad", synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.02))
             if M else None, M) for i, M in enumerate(shapes)]
    x = synth.activations(20, N, 0, N, K)
    ys = run_group(mats, K, x)
    for (w, M), y in zip(mats, ys):
        if M:
            assert_products(y, w, M, K, x, REL_F32, what="group M=%d N=%d" % (M, N))


def test_mat_vec_group_many_items_chunks_and_matches_single():
    rng = np.random.default_rng(31)
    K, N = 512, 1
    Ms = [int(m) for m in rng.integers(1, 300, size=70)]
    mats = [(synth.weight(21, i, 0, M, K, "tern", synth.ScaleDist("uniform", 0.01, 0.1)), M)
            for i, M in enumerate(Ms)]
    x = synth.activations(21, 0, 0, N, K)
    ys = run_group(mats, K, x)
    for (w, M), y in zip(mats, ys):
        assert_products(y, w, M, K, x, REL_F32, what="many M=%d" % M)
    # grouping does not change results: the same matrix alone in a group of one
    for (w, M), y in list(zip(mats, ys))[:5]:
        (y1,) = run_group([(w, M)], K, x)
        assert np.array_equal(y1, y)


def test_mat_vec_group_mixed_eligibility():
    """K/64 % 8 != 0 rows (not 16-byte aligned) take the generic kernel inside a group."""
    K, N = 64 * 12, 3
    mats = [(synth.weight(22, i, 0, M, K, "quad", synth.ScaleDist("uniform", 0.01, 0.1)), M)
            for i, M in enumerate([100, 2000, 5])]
    x = synth.activations(22, 0, 0, N, K)
    for (w, M), y in zip(mats, run_group(mats, K, x, ldx=K + 5)):
        assert_products(y, w, M, K, x, REL_F32, what="mixed M=%d" % M)


@pytest.mark.parametrize("N", [1, 3, 8])
def test_mat_vec_stream_path_full_oracle(N):
    """M large enough for the whole-K streaming kernel on a single call; every row checked."""
    M, K = 20000 + 7, 1024
    w = synth.weight(23, N, 0, M, K, "quad", synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.01))
    x = synth.activations(23, N, 0, N, K)
    y = run_mat_vec(dev(w), M, K, x, ldy=M + 9)
    assert_products(y, w, M, K, x, REL_F32, what="stream N=%d" % N)


# The streaming kernel across K (1, 2, 4, 6, 8 and 12 stages of 16 blocks per row, and two
# stages plus a half stage at K = 2560, where K/64 = 8 mod 16) and N, with ragged M so that
# the last tile is partial; every row checked.
@pytest.mark.parametrize("K,N", [(1024, 1), (2048, 1), (2048, 4), (2560, 3), (4096, 1), (4096, 2), (4096, 4),
                                 (6144, 2), (8192, 1), (12288, 1), (12288, 2)])
def test_mat_vec_stream_across_k(K, N):
    M = 16384 + 5
    w = synth.weight(24, K // 64, N, M, K, "tern_c3", synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.01))
    x = synth.activations(24, K // 64, N, N, K)
    y = run_mat_vec(dev(w), M, K, x, ldy=M + 3)
    assert_products(y, w, M, K, x, REL_F32, what="stream K=%d N=%d" % (K, N))


@pytest.mark.parametrize("K,N", [(4096, 1), (12288, 1), (4096, 2)])
def test_mat_vec_stream_nonfinite_activation(K, N):
    """An inf or NaN activation makes every output of its column non-finite, as in the
    oracle (a zero weight times inf is NaN); the other column stays within tolerance."""
    M = 16384 + 5
    w = synth.weight(26, K // 64, N, M, K, "tern_c3", synth.ScaleDist("uniform", 0.005, 0.05))
    x = synth.activations(26, K // 64, N, N, K)
    x[0, 100] = np.inf
    if N == 2:
        x[0, 7] = np.nan
    y = run_mat_vec(dev(w), M, K, x, ldy=M + 3)
    rows = np.arange(0, M, 7)
    y_ref, bound = oracle.mul_mat(w, M, K, x, rows=rows)
    assert not np.isfinite(y_ref[0]).any()
    assert not np.isfinite(y[0]).any(), "column with an inf activation gave finite outputs"
    if N == 2:
        assert np.isfinite(y[1]).all()
        r = oracle.check_products(y[1:, rows], y_ref[1:], bound[1:], REL_F32)
        assert r["ok"], r


@pytest.mark.parametrize("K", [4096, 12288])
def test_mat_vec_stream_blocks_of_far_apart_magnitudes(K):
    """Each 64-weight block of the activation scaled by its own power of ten, 1e-30 .. 1e30:
    the per-block (N = 1, K <= 8192) and per-column staging both meet the bound."""
    M, N = 16384 + 5, 1
    w = synth.weight(27, K // 64, N, M, K, "quad", synth.ScaleDist("uniform", 0.005, 0.05))
    x = synth.activations(27, K // 64, N, N, K)
    rng = np.random.default_rng(27)
    x *= (10.0 ** rng.integers(-30, 31, K // 64)).repeat(64).astype(np.float32)[None, :]
    y = run_mat_vec(dev(w), M, K, x)
    assert_products(y, w, M, K, x, REL_F32, rows=np.arange(0, M, 3), what="far-apart blocks K=%d" % K)


def test_mat_vec_group_ragged_members_long_rows():
    """Group members whose row counts leave partial tiles, at K = 12288 (12 stages a row)."""
    K, N = 12288, 1
    Ms = (16384 + 1, 3, 2 + 16, 1000 + 7)
    mats = [(synth.weight(25, i, 0, M, K, "quad", synth.ScaleDist("uniform", 0.005, 0.05)), M)
            for i, M in enumerate(Ms)]
    x = synth.activations(25, 0, 1, N, K)
    for (w, M), y in zip(mats, run_group(mats, K, x)):
        assert_products(y, w, M, K, x, REL_F32, what="group M=%d" % M)


def test_mat_vec_group_stack_8b_layer_workload():
    wl = synth.STACK_8B
    K = 4096
    names = ["q", "k", "v", "o", "gate", "up"]
    mats = [(ws(wl, n, layer=1), wl.shapes[n][0]) for n in names]
    x = synth.activations(wl.seed, 0, synth.stack_x_matrix_index(K), 1, K)
    rng = np.random.default_rng(7)
    for (w, M), y, n in zip(mats, run_group(mats, K, x), names):
        rows = np.unique(np.concatenate([rng.integers(0, M, 256), [0, M - 1]]))
        assert_products(y, w, M, K, x, REL_F32, rows=rows, what=n)


# =============================================================================== grouped GEMM

def run_gemm_group(mats, K, x, precision):
    torch = _torch()
    N = x.shape[0]
    xd = dev(x)
    keep, entries, ys = [], [], []
    for w, M in mats:
        wd = dev(w) if M else None
        yd = torch.full((N, M + 5), float("nan"), dtype=torch.float32, device="cuda")
        keep.append(wd)
        ys.append(yd)
        entries.append((wd.data_ptr() if wd is not None else 0, M, yd.data_ptr(), M + 5))
    items = B.make_items(entries)
    need = B.mul_mat_group_workspace_bytes(items, len(entries), K, N, precision)
    wsd = torch.full((max(need, 16) // 4 + 1,), float("nan"), dtype=torch.float32, device="cuda")
    st = B.mul_mat_group_raw(items, len(entries), K, xd.data_ptr(), K, N, precision, wsd.data_ptr(), need,
                             torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().q2_0_status_string(st)
    out = []
    for (w, M), yd in zip(mats, ys):
        y = host(yd)
        assert np.all(np.isnan(y[:, M:])), "group GEMM wrote past M"
        out.append(y[:, :M])
    return out


@pytest.mark.parametrize("precision,rel", [(B.Q2_0_PREC_F16_MFMA, REL_F16), (B.Q2_0_PREC_F32, REL_F32),
                                             (B.Q2_0_PREC_F32_MFMA, REL_F32)])
@pytest.mark.parametrize("Ms,K,N", [((4096 // 8, 1024 // 8, 1024 // 8), 2048, 96), ((300, 0, 77, 129), 576, 130),
                                    ((64,) * 20, 192, 64), ((1000, 24), 4096, 9)])
def test_mul_mat_group_matches_oracle(precision, rel, Ms, K, N):
    mats = [(synth.weight(17, i, len(Ms), M, K, "quad", synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.02)), M)
            for i, M in enumerate(Ms)]
    x = synth.activations(17, len(Ms), K, N, K)
    ys = run_gemm_group(mats, K, x, precision)
    for (w, M), y in zip(mats, ys):
        if M:
            assert_products(y, w, M, K, x, rel, what="group item M=%d K=%d N=%d" % (M, K, N))


def test_mul_mat_group_gate_up_8b_full_size():
    """The 8B stack's gate/up pair at N = 512 (768 tiles of 128 x 128, no K split: one
    round at three workgroups per CU); sampled rows of both, run to run bit-equal."""
    wl = synth.STACK_8B
    names = ["gate", "up"]
    K = wl.shapes["gate"][1]
    mats = [(ws(wl, n, layer=0), wl.shapes[n][0]) for n in names]
    x = synth.activations(wl.seed, 0, synth.stack_x_matrix_index(K) + 11, 512, K)
    a = run_gemm_group(mats, K, x, B.Q2_0_PREC_F16_MFMA)
    b = run_gemm_group(mats, K, x, B.Q2_0_PREC_F16_MFMA)
    for (w, M), ya, yb, n in zip(mats, a, b, names):
        assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32)), "run-to-run difference in " + n
        rows = np.unique(np.concatenate([np.arange(0, M, 61), np.arange(M - 40, M)]))
        assert_products(ya, w, M, K, x, REL_F16, rows=rows, what="gate/up " + n)


def test_mul_mat_256_row_tiles_ragged():
    """256-row tiles (chosen for 1024 of them in two full rounds) with a partial last row
    tile (M = 65357), a partial column tile (N = 500) and a padded last step group
    (K / 64 = 10 blocks)."""
    M, K, N = 65357, 640, 500
    w = synth.weight(29, M, N, M, K, "quad", synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.02))
    x = synth.activations(29, M, N, N, K)
    y = run_mul_mat(dev(w), M, K, x, B.Q2_0_PREC_F16_MFMA, ldy=M + 3)
    rows = np.unique(np.concatenate([np.arange(0, M, 29), np.arange(M - 300, M)]))
    assert_products(y, w, M, K, x, REL_F16, rows=rows, what="256-row tiles M=%d K=%d N=%d" % (M, K, N))


def test_mul_mat_group_prefill_qkv_deterministic():
    wl = synth.PREFILL_1P7B
    names = ["q", "k", "v"]
    K = wl.shapes["q"][1]
    mats = [(ws(wl, n), wl.shapes[n][0]) for n in names]
    x = synth.activations(wl.seed, 0, 0, 512, K)
    a = run_gemm_group(mats, K, x, B.Q2_0_PREC_F16_MFMA)
    b = run_gemm_group(mats, K, x, B.Q2_0_PREC_F16_MFMA)
    for (w, M), ya, yb, n in zip(mats, a, b, names):
        assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32)), "run-to-run difference in " + n
        rows = np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
        assert_products(ya, w, M, K, x, REL_F16, rows=rows, what="qkv " + n)
