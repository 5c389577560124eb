"""How v_mfma_f32_32x32x16_f16 rounds, as far as the fp32-grade GEMM's error bound counts on it.

Q2_0_PREC_F32_MFMA sums each pair of blocks in one f32 accumulator over 8 MFMAs and
bounds the error by counting at most 4 f32 roundings per MFMA (include/q2_0.h, its
1e-5 contract).  These one-wave probes (every row of A and column of B the same, so all
1024 results are equal) pin what that count rests on:
  * the fp16 products are exact and small ones are not dropped one by one: 1 + 15 * 2^-24
    and 1 + 16 * 2^-24 come out as the correctly rounded exact sums;
  * the 16 products reach the accumulator in groups of at least 8 (at most two roundings):
    sixteen products of 1 on an accumulator of 2^26 (spacing 8) are all kept, which groups
    of 4 or fewer (each a tie, rounded to even) would lose.
"""

import ctypes
import os

import numpy as np
import pytest

from ternary_bit_quantized_amd import build

pytestmark = pytest.mark.gpu


def probe(a, b, c):
    torch = __import__("torch")
    lib = ctypes.CDLL(build.CEIL_LIB)
    lib.q2_0_probe_mfma_f16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p]
    at = torch.tensor(np.asarray(a, dtype=np.float16), device="cuda")
    bt = torch.tensor(np.asarray(b, dtype=np.float16), device="cuda")
    assert at.numel() == 16 and bt.numel() == 16
    out = torch.full((1024,), float("nan"), dtype=torch.float32, device="cuda")
    assert lib.q2_0_probe_mfma_f16(at.data_ptr(), bt.data_ptr(), float(c), out.data_ptr()) == 0
    r = out.cpu().numpy()
    assert np.all(r == r[0]), "results differ between lanes"
    return np.float64(r[0])


def test_library_present():
    assert os.path.exists(build.CEIL_LIB), "libq2_0_ceilings.so is not built"


def test_products_exact_and_small_ones_not_dropped():
    s = 2.0 ** -12
    # 1 + 15 * 2^-24: the exact sum rounds (tie, to even) to 1 + 2^-20
    assert probe([1.0] + [s] * 15, [1.0] + [s] * 15, 0.0) == 1.0 + 2.0 ** -20
    # 1 + 16 * 2^-24 = 1 + 2^-20 exactly
    assert probe([s] * 16, [s] * 16, 1.0) == 1.0 + 2.0 ** -20
    # 16 (1 + 2^-10)^2 = 16 + 2^-5 + 2^-16, exact in f32
    assert probe([1 + 2.0 ** -10] * 16, [1 + 2.0 ** -10] * 16, 0.0) == 16.0 + 2.0 ** -5 + 2.0 ** -16


def test_products_reach_the_accumulator_in_groups_of_at_least_eight():
    ones = [1.0] * 16
    for j in range(0, 4):   # spacing 2^j <= 8: the +16 survives any grouping of >= 8
        c = 2.0 ** (23 + j)
        assert probe(ones, ones, c) == c + 16.0, "C = 2^%d" % (23 + j)
