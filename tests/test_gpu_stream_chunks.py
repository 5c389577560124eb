"""The N >= 3 streaming mat-vec on a K whose activation does not fit in LDS: consecutive
launches over chunks of whole 16-block stages, the first writing y and the others adding
to it.  Against the fp64 oracle on the single, group and batch entry points:

  * K = 6144, 6656 (a last chunk of 8 blocks at N = 8: a half stage), 12288 and 16384 at
    N = 3, 5 and 8 (N = 3: whole K at 6144, chunks of 64-128 blocks beyond; N = 5:
    48-64; N = 8: 48), ragged M, strided x and y;
  * y past M untouched (the added chunks read and write only their own rows);
  * run-to-run bitwise determinism;
  * a grouped call of smaller matrices (their long K takes the K-split kernel) and a
    batch with two activations (the Qwen3-1.7B decode's K = 2048 and 6144 at N = 8),
    whose large K = 6144 item is chunked and whose small one is not.
"""

import numpy as np
import pytest

from ternary_bit_quantized_amd import q2_0 as B
from ternary_bit_quantized_amd import synth
from test_gpu_parity import REL_F32, assert_products, dev, host, run_group, run_mat_vec
from test_gpu_batch import run_batch

pytestmark = pytest.mark.gpu


def sample_rows(M, step=61):
    return np.unique(np.concatenate([np.arange(0, M, step), np.arange(max(0, M - 20), M)]))


def wgt(seed, M, K):
    return synth.weight(300 + seed, K // 64, M, M, K, "tern_c3", synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.01))


@pytest.mark.parametrize("K", [6144, 6656, 12288, 16384])
@pytest.mark.parametrize("N", [3, 5, 8])
def test_chunked_stream_long_k(K, N):
    M = 16384 + 5
    w = wgt(K % 101 + N, M, K)
    x = synth.activations(301, K // 64, N, N, K)
    y = run_mat_vec(dev(w), M, K, x, ldx=K + 4, ldy=M + 3)
    assert_products(y, w, M, K, x, REL_F32, rows=sample_rows(M), what="chunked K=%d N=%d" % (K, N))


def test_chunked_stream_leaves_y_past_m_and_is_deterministic():
    torch = __import__("torch")
    M, K, N = 16384 + 9, 12288, 8
    w = dev(wgt(7, M, K))
    x = dev(synth.activations(302, 0, 0, N, K))
    outs = []
    for _ in range(2):
        y = torch.full((N, M + 5), float("nan"), dtype=torch.float32, device="cuda")
        st = B.mul_mat_vec_raw(w.data_ptr(), M, K, x.data_ptr(), K, N, y.data_ptr(), M + 5,
                               torch.cuda.current_stream().cuda_stream)
        assert st == 0
        yh = host(y)
        assert np.all(np.isnan(yh[:, M:])), "wrote past M"
        assert not np.any(np.isnan(yh[:, :M]))
        outs.append(yh[:, :M].copy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


def test_chunked_stream_group():
    N, K = 5, 6144
    mats = [(wgt(11, 3000, K), 3000, None), (wgt(12, 2048, K), 2048, None)]
    x = synth.activations(303, 0, 0, N, K)
    ys = run_group([(w, M) for (w, M, c) in mats], K, x)
    for (w, M, _), y in zip(mats, ys):
        assert_products(y, w, M, K, x, REL_F32, what="chunked group M=%d" % M)


def test_chunked_stream_batch_two_activations():
    N = 8
    Ks = (2048, 6144)
    xs_h = [synth.activations(304, i, 0, N, K) for i, K in enumerate(Ks)]
    xs = [dev(x) for x in xs_h]
    products = [(wgt(20 + i, M, K), M, K, xi) for i, (M, K, xi) in
                enumerate([(6144, 2048, 0), (2048, 2048, 0), (20000, 6144, 1), (2048, 6144, 1)])]
    for (w, M, K, xi), y in zip(products, run_batch(products, xs, N)):
        assert_products(y, w, M, K, xs_h[xi], REL_F32, rows=sample_rows(M), what="batch M=%d K=%d" % (M, K))
