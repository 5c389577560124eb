"""The streaming mat-vec with the activation staged in windows (rows of any K) and the
batched entry point whose items each carry their own K and activation, against the fp64
oracle.

  * K from 7168 to 16384 at N = 1 and 2: two and three windows, a ragged half stage in the
    last window (K / 64 = 136), 16-row tiles whose windows fall to different waves, and
    (fewer rows, smaller workgroups) whole rows in one window;
  * q2_0_mul_mat_vec_batch: a decode-step-like batch (K = 4096 and 12288 activations, a
    vocabulary-sized head), more than eight activations (several launches), more than 64
    items, items the fast kernels cannot take in the middle, and 16-bit activations;
  * a matrix whose tiles per workgroup would overflow the LDS accumulator of the windowed
    path, so that the launch takes more workgroups than the GPU holds at once.
"""

import numpy as np
import pytest

import oracle
from ternary_bit_quantized_amd import q2_0 as B
from ternary_bit_quantized_amd import synth
from test_gpu_parity import REL_F32, assert_products, dev, host, run_mat_vec

pytestmark = pytest.mark.gpu


def tern(seed, M, K, codes="tern_c3"):
    return synth.weight(80 + seed, M, K // 64, M, K, codes, synth.ScaleDist("uniform", 0.005, 0.05))


def sample_rows(M, step=53):
    return np.unique(np.concatenate([np.arange(0, M, step), np.arange(max(0, M - 20), M)]))


@pytest.mark.parametrize("K", [7168, 8704, 12288, 16384])
@pytest.mark.parametrize("N", [1, 2])
@pytest.mark.parametrize("M", [16400, 4100, 1000])
def test_windowed_mat_vec_long_rows(K, N, M):
    """M = 16400: 16-wave workgroups, rows in windows of at most 6 stages; 4100 and 1000:
    8- and 4-wave workgroups, whose LDS holds a whole row of up to 13 and 16 stages."""
    w = tern(K % 97, M, K)
    x = synth.activations(81, K, N, N, K)
    y = run_mat_vec(dev(w), M, K, x)
    assert_products(y, w, M, K, x, REL_F32, rows=sample_rows(M), what="K=%d N=%d" % (K, N))


def test_windowed_mat_vec_deterministic():
    M, K = 20000, 12288
    w = tern(3, M, K)
    x = synth.activations(82, 0, 0, 1, K)
    wd = dev(w)
    a = run_mat_vec(wd, M, K, x)
    b = run_mat_vec(wd, M, K, x)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def run_batch(products, xs, N, xt=B.Q2_0_ACT_F32):
    """products: [(w host bytes, M, K, x index)]; xs: device activation tensors.  Returns [y_i]."""
    torch = __import__("torch")
    keep, entries, ys = [], [], []
    for w, M, K, xi in products:
        wd = dev(w) if M else None
        yd = torch.full((N, M + 3), float("nan"), dtype=torch.float32, device="cuda")
        keep.append(wd)
        ys.append(yd)
        x = xs[xi]
        entries.append((wd.data_ptr() if wd is not None else 0, M, K, x.data_ptr(), x.shape[1], yd.data_ptr(),
                        M + 3))
    items = B.make_batch_items(entries)
    st = B.mul_mat_vec_batch_raw(items, len(entries), xt, N, torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().q2_0_status_string(st)
    out = []
    for (w, M, K, xi), yd in zip(products, ys):
        y = host(yd)
        assert np.all(np.isnan(y[:, M:])), "batch wrote past M"
        out.append(y[:, :M])
    return out


@pytest.mark.parametrize("N", [1, 2])
def test_batch_decode_step_like(N):
    """Three activations (K = 2048, 6144 and a second one at 2048), seven matrices of each
    layer shape of a small model, and a head: one launch, mixed K, mixed windows."""
    xs_h = [synth.activations(83, i, 0, N, K) for i, K in enumerate((2048, 6144, 2048))]
    xs = [dev(x) for x in xs_h]
    shapes = [(2048, 2048, 0), (1024, 2048, 0), (1024, 2048, 0), (2048, 2048, 2), (6144, 2048, 2),
              (6144, 2048, 2), (2048, 6144, 1), (30000, 2048, 0)]
    products = [(tern(10 + i, M, K), M, K, xi) for i, (M, K, xi) in enumerate(shapes)]
    for (w, M, K, xi), y in zip(products, run_batch(products, xs, N)):
        rows = None if M < 3000 else sample_rows(M)
        assert_products(y, w, M, K, xs_h[xi], REL_F32, rows=rows, what="batch M=%d K=%d" % (M, K))


def test_batch_many_activations_and_items():
    """Twelve activations (more than one launch holds) and 70 items (more than 64), some with
    rows the fast kernels cannot take (K / 64 % 8 != 0), some empty."""
    N = 1
    Ks = [512, 1024, 1536, 640, 2048, 512, 4096, 576, 1024, 3072, 512, 8192]
    xs_h = [synth.activations(84, i, 0, N, K) for i, K in enumerate(Ks)]
    xs = [dev(x) for x in xs_h]
    rng = np.random.default_rng(85)
    products = []
    for i in range(70):
        xi = min(i // 6, len(Ks) - 1)
        K = Ks[xi]
        M = 0 if i % 17 == 5 else int(rng.integers(1, 700))
        products.append((tern(100 + i, M, K) if M else None, M, K, xi))
    for (w, M, K, xi), y in zip(products, run_batch(products, xs, N)):
        if M:
            assert_products(y, w, M, K, xs_h[xi], REL_F32, what="item M=%d K=%d" % (M, K))


def test_batch_f16_activations_bitwise_equal_f32():
    torch = __import__("torch")
    N = 2
    Ks = (2048, 12288)
    xs32 = [synth.to_f16(synth.activations(86, i, 0, N, K)).astype(np.float32) for i, K in enumerate(Ks)]
    products = [(tern(200 + i, M, K), M, K, xi) for i, (M, K, xi) in
                enumerate([(3000, 2048, 0), (17000, 12288, 1), (500, 2048, 0)])]
    a = run_batch(products, [dev(x) for x in xs32], N)
    b = run_batch(products, [dev(x).to(torch.float16) for x in xs32], N, B.Q2_0_ACT_F16)
    for ya, yb in zip(a, b):
        assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32))


@pytest.mark.parametrize("N", [1, 2])
def test_windowed_mat_vec_more_workgroups_than_the_gpu_holds(N):
    """~44000 tiles of 12288-long rows: at 256 workgroups each would hold more tiles than
    the LDS accumulator of the windowed path, so the launch takes more workgroups."""
    torch = __import__("torch")
    M, K = 700000 if N == 2 else 1200000, 12288
    nb = K // 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(87 + N)
    wd = torch.randint(0, 256, (M, nb, 18), dtype=torch.uint8, device="cuda", generator=gen)
    wd[:, :, 1] = 0x20 + (wd[:, :, 1] & 0x0F)       # scales: normal halves of moderate size
    x = synth.activations(87, N, 0, N, K)
    y = run_mat_vec(wd.view(M, nb * 18), M, K, x)
    rows = np.unique(np.concatenate([np.arange(0, M, 4099), np.arange(M - 16, M)]))
    w_rows = host(wd.view(M, nb * 18)[torch.from_numpy(rows).cuda()])
    y_ref, bound = oracle.mul_mat(w_rows, rows.size, K, x)
    r = oracle.check_products(y[:, rows], y_ref, bound, REL_F32)
    assert r["ok"], r
