"""q2_0_mul_mat_noalloc (static scratch) against q2_0_mul_mat (caller workspace).

Both run the same kernels with the same plan, so their results must agree bit for bit;
each call is also checked against the oracle.  Two calls in a row, the second smaller,
show that the shared scratch carries nothing from one call into the next.
"""

import numpy as np
import pytest

from ternary_bit_quantized_amd import q2_0 as B
from ternary_bit_quantized_amd import synth
from test_gpu_parity import REL_F16, REL_F32, assert_products, dev, host, run_mul_mat

pytestmark = pytest.mark.gpu


def run_noalloc(w_d, M, K, x, precision):
    torch = __import__("torch")
    N = x.shape[0]
    xd = dev(x)
    yd = torch.full((N, M + 3), float("nan"), dtype=torch.float32, device="cuda")
    st = B.mul_mat_noalloc_raw(w_d.data_ptr(), M, K, xd.data_ptr(), K, N, yd.data_ptr(), M + 3, precision,
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().q2_0_status_string(st)
    y = host(yd)
    assert np.all(np.isnan(y[:, M:])), "wrote past M"
    return y[:, :M]


# (M, K, N) pairs run back to back: a call with a K split and partials in the scratch,
# then a smaller one; then the smaller first and a larger one
CASES = [((4096, 12288, 512), (300, 2048, 130)),
         ((2048, 4096, 96), (4096, 4096, 512)),
         ((1024, 4096, 64), (1000, 1024, 9))]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_mul_mat_two_calls(first, second):
    for i, (M, K, N) in enumerate((first, second)):
        w = synth.weight(71, i, M, M, K, "tern", synth.ScaleDist("uniform", 0.002, 0.02))
        x = synth.activations(71, i, M, N, K)
        wd = dev(w)
        a = run_noalloc(wd, M, K, x, B.Q2_0_PREC_F16_MFMA)
        b = run_mul_mat(wd, M, K, x, B.Q2_0_PREC_F16_MFMA)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "call %d (%d, %d, %d)" % (i, M, K, N)
        rows = np.unique(np.concatenate([np.arange(0, M, 29), [M - 1]]))
        assert_products(a, w, M, K, x, REL_F16, rows=rows, what="noalloc call %d" % i)


@pytest.mark.parametrize("N,precision,rel", [(4, B.Q2_0_PREC_F16_MFMA, REL_F32), (40, B.Q2_0_PREC_F32, REL_F32)])
def test_noalloc_paths_without_scratch(N, precision, rel):
    """Calls that need no scratch (the mat-vec, the fp32 GEMM) pass straight through."""
    M, K = 500, 2048
    w = synth.weight(72, N, precision, M, K, "tern", synth.ScaleDist("uniform", 0.002, 0.02))
    x = synth.activations(72, N, precision, N, K)
    wd = dev(w)
    a = run_noalloc(wd, M, K, x, precision)
    b = run_mul_mat(wd, M, K, x, precision)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert_products(a, w, M, K, x, rel, what="noalloc N=%d" % N)
