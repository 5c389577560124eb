"""CPU models of how the fast kernels carry the activations, against the accuracy
statements of include/q2_0.h.

The products of the fast paths are exact (fp16 or small-integer operands into f32),
so their error budget is what happens to x on the way into the matrix cores plus f32
summation.  These tests rebuild each staging in numpy, element by element, and check:
  * the per-element error bounds stated in the header;
  * that the header's range condition keeps the staging error inside the budget that
    the stated tolerance leaves after f32 summation;
  * that without the condition the tolerance can indeed fail (so the condition is not
    vacuous).

Stagings (what the kernels do; numpy's float16 conversion is IEEE nearest-even with
subnormals, as is the GPU's):
  * fp16 GEMM: column scaled by 2^e so that its max |x| is in [2^14, 2^15), one fp16;
  * hi/lo (mat-vec, N > 1 or the K-split kernel): the same scaling, x = hi + lo with
    hi = fp16(v), lo = fp16(v - hi);
  * limbs (mat-vec, N = 1): each 64-element block scaled by 2^e so that its max |x| is
    in [2^10, 2^11), then four limbs L = rint(w), w = (w - L) * 2^11, in f32.
"""

import numpy as np
import pytest

F32 = np.float32


def pow2_exponent(amax, top):
    """e with amax * 2^e in [2^(top-1), 2^top); 0 for zero or non-finite amax."""
    if not (amax > 0) or not np.isfinite(amax):
        return 0
    return top - int(np.frexp(amax)[1])


def stage_f16(x):
    """fp16 GEMM staging of one column (f32 in, the value the MFMA sees, as float64)."""
    e = pow2_exponent(float(np.max(np.abs(x))), 15)
    v = (x.astype(F32) * F32(2.0 ** e)).astype(F32)
    return v.astype(np.float16).astype(np.float64) * 2.0 ** -e


def stage_hilo(x):
    e = pow2_exponent(float(np.max(np.abs(x))), 15)
    v = (x.astype(F32) * F32(2.0 ** e)).astype(F32)
    hi = v.astype(np.float16)
    lo = (v - hi.astype(F32)).astype(F32).astype(np.float16)
    return (hi.astype(np.float64) + lo.astype(np.float64)) * 2.0 ** -e


def stage_limbs(x):
    out = np.empty(x.shape, dtype=np.float64)
    for b in range(0, x.size, 64):
        blk = x[b:b + 64].astype(F32)
        e = pow2_exponent(float(np.max(np.abs(blk))), 11)
        w = (blk * F32(2.0 ** e)).astype(F32)
        acc = np.zeros(blk.size)
        for l in range(4):
            L = np.rint(w).astype(F32)
            w = ((w - L) * F32(2048.0)).astype(F32)
            acc += L.astype(np.float64) * 2.0 ** (-11 * l)
        out[b:b + 64] = acc * 2.0 ** -e
    return out


def rng(seed):
    return np.random.default_rng(np.random.SeedSequence([2024, seed]))


def column_with_range(seed, K, decades):
    """N(0,1) scaled by 10^u, u uniform in [-decades, 0]: wide dynamic range."""
    r = rng(seed)
    return (r.standard_normal(K) * 10.0 ** r.uniform(-decades, 0, K)).astype(F32)


@pytest.mark.parametrize("seed", range(6))
def test_element_bounds_fp16_and_hilo(seed):
    x = column_with_range(seed, 4096, 14)
    cmax = float(np.max(np.abs(x)))
    xd = x.astype(np.float64)
    err16 = np.abs(stage_f16(x) - xd)
    assert np.all(err16 <= np.maximum(2.0 ** -11 * np.abs(xd), 2.0 ** -39 * cmax))
    # elements within 2^28 of the column maximum stay fp16 normals: pure relative error
    big = np.abs(xd) >= 2.0 ** -28 * cmax
    assert np.all(err16[big] <= 2.0 ** -11 * np.abs(xd[big]))
    errhl = np.abs(stage_hilo(x) - xd)
    assert np.all(errhl <= np.maximum(2.0 ** -22 * np.abs(xd), 2.0 ** -39 * cmax))
    near = np.abs(xd) >= 2.0 ** -17 * cmax
    assert np.all(errhl[near] <= 2.0 ** -22 * np.abs(xd[near]))


@pytest.mark.parametrize("seed", range(6))
def test_element_bounds_limbs(seed):
    x = column_with_range(seed + 10, 4096, 9)
    xd = x.astype(np.float64)
    err = np.abs(stage_limbs(x) - xd)
    bmax = np.repeat(np.max(np.abs(xd).reshape(-1, 64), axis=1), 64)
    assert np.all(err <= 2.0 ** -44 * bmax)
    near = np.abs(xd) >= 2.0 ** -20 * bmax
    assert np.all(err[near] == 0.0), "elements within 2^20 of their block maximum must be exact"


def weights_with_zero_column(seed, M, K, k0):
    r = rng(100 + seed)
    q = r.integers(0, 3, size=(M, K)).astype(np.float64)
    q[:, k0] = 1
    d = r.uniform(0.005, 0.05, size=(M, K // 64)).astype(np.float16).astype(np.float64)
    return (q - 1) * np.repeat(d, 64, axis=1)


def staging_error_ratio(stage, W, x, k0, big):
    """max over rows of |W (staged x - x)| / A and the rows' max |x| * sum|W| / A."""
    x = x.copy()
    x[k0] = big
    xd = x.astype(np.float64)
    A = np.abs(W) @ np.abs(xd)
    err = np.abs(W @ (stage(x) - xd))
    cond = float(np.max(np.abs(xd))) * np.abs(W).sum(axis=1) / A
    return float(np.max(err / A)), float(np.max(cond))


@pytest.mark.parametrize("stage,rel,budget,cpow", [
    # (staging, tolerance, f32 summation allowance at K <= 16384, header's 2^c)
    (stage_f16, 2e-3, 16384 * 2.0 ** -24, 28),
    (stage_hilo, 1e-5, 100 * 2.0 ** -24, 21),
    (stage_limbs, 1e-5, 100 * 2.0 ** -24, 21),
])
def test_range_condition_keeps_staging_inside_the_budget(stage, rel, budget, cpow):
    """At the edge of the range condition (a zero-weighted outlier as large as the
    condition allows) the modelled staging error stays below the tolerance minus the
    f32 summation allowance."""
    M, K, k0 = 64, 4096, 3 * 64 + 17
    W = weights_with_zero_column(1, M, K, k0)
    x = rng(7).standard_normal(K).astype(F32)
    x[k0] = 0
    A = np.abs(W) @ np.abs(x.astype(np.float64))
    big = F32(0.999 * 2.0 ** cpow * float(np.min(A / np.abs(W).sum(axis=1))))
    ratio, cond = staging_error_ratio(stage, W, x, k0, big)
    assert cond <= 2.0 ** cpow
    assert ratio <= rel - budget, "staging error %.3g of A exceeds the budget" % ratio


@pytest.mark.parametrize("stage,rel,big", [(stage_f16, 2e-3, 2.0 ** 42), (stage_hilo, 1e-5, 2.0 ** 32)])
def test_range_condition_is_needed(stage, rel, big):
    """Far outside the condition a zero-weighted outlier pushes the live activations into
    fp16's subnormal range or below it, and the tolerance fails: the header cannot drop
    the condition for these stagings."""
    M, K, k0 = 64, 4096, 3 * 64 + 17
    W = weights_with_zero_column(2, M, K, k0)
    x = rng(8).standard_normal(K).astype(F32)
    ratio, cond = staging_error_ratio(stage, W, x, k0, F32(big))
    assert cond > 2.0 ** 30
    assert ratio > rel


def test_limbs_tolerate_far_larger_outliers_than_hilo():
    """The N = 1 limb staging scales per 64-element block, so an outlier only affects its
    own block: an outlier 2^32 above the rest that breaks hi/lo keeps limbs in budget
    when it sits in a block of its own... and even inside a live block stays within
    2^-44 of that block's maximum."""
    M, K, k0 = 64, 4096, 3 * 64 + 17
    W = weights_with_zero_column(3, M, K, k0)
    x = rng(9).standard_normal(K).astype(F32)
    ratio, _ = staging_error_ratio(stage_limbs, W, x, k0, F32(2.0 ** 32))
    assert ratio <= 1e-5 - 100 * 2.0 ** -24


def f32_mfma_model(W16, x):
    """Q2_0_PREC_F32_MFMA for one column: W16 (M x K, the fp16 values d*(q-1)) times x staged
    as hi/lo, every product exact; each 16-k step's products reach the f32 accumulator as
    two exactly summed groups of 8 (the behaviour measured on the matrix cores), hi step
    then lo step; the accumulator restarts every 128 k and is added into fp64; one
    rounding to f32 at the end (after the exact power-of-two unscaling)."""
    e = pow2_exponent(float(np.max(np.abs(x))), 15)
    v = (x.astype(F32) * F32(2.0 ** e)).astype(F32)
    hi = v.astype(np.float16).astype(np.float64)
    lo = (v - v.astype(np.float16).astype(F32)).astype(F32).astype(np.float16).astype(np.float64)
    Ph, Pl = W16 * hi, W16 * lo                     # exact: 11-bit by 11-bit significands
    M, K = W16.shape
    mst = np.zeros(M)
    acc = np.zeros(M, dtype=F32)
    for k0 in range(0, K, 16):
        for P in (Ph, Pl):
            for g in (0, 8):
                acc = (acc.astype(np.float64) + P[:, k0 + g:k0 + g + 8].sum(axis=1)).astype(F32)
        if (k0 + 16) % 128 == 0 or k0 + 16 == K:
            mst += acc.astype(np.float64)
            acc = np.zeros(M, dtype=F32)
    return (mst * 2.0 ** -e).astype(F32)


@pytest.mark.parametrize("K", [4096, 16384])
def test_f32_mfma_model_meets_its_bound_at_the_range_limit(K):
    """The whole arithmetic of Q2_0_PREC_F32_MFMA, modelled, stays within 1e-5 * A with a
    zero-weighted outlier at the edge of its range condition (2^21), and on plain data.
    (The header's budget counts 4 roundings per MFMA; this model takes the measured 2.)"""
    M, k0 = 48, 3 * 64 + 17
    W = weights_with_zero_column(4, M, K, k0)
    W16 = W.astype(np.float16).astype(np.float64)
    assert np.array_equal(W16, W)                   # d*(q-1) is exact in fp16
    x = rng(10).standard_normal(K).astype(F32)
    x[k0] = 0
    A0 = np.abs(W) @ np.abs(x.astype(np.float64))
    for big in (0.0, 1e4, 0.999 * 2.0 ** 21 * float(np.min(A0 / np.abs(W).sum(axis=1)))):
        xb = x.copy()
        xb[k0] = F32(big)
        xd = xb.astype(np.float64)
        A = np.abs(W) @ np.abs(xd)
        err = np.abs(f32_mfma_model(W16, xb).astype(np.float64) - W @ xd)
        assert float(np.max(err / A)) <= 1e-5, "outlier %.3g: %.3g" % (big, float(np.max(err / A)))


def test_f32_mfma_model_needs_the_range_condition():
    """Far outside the condition (a zero-weighted outlier 2^36 above the rest) the lo
    halves of the live activations fall below fp16's subnormals and the bound fails."""
    M, K, k0 = 48, 4096, 3 * 64 + 17
    W = weights_with_zero_column(5, M, K, k0)
    x = rng(11).standard_normal(K).astype(F32)
    x[k0] = F32(2.0 ** 36)
    xd = x.astype(np.float64)
    A = np.abs(W) @ np.abs(xd)
    err = np.abs(f32_mfma_model(W.astype(np.float16).astype(np.float64), x).astype(np.float64) - W @ xd)
    assert float(np.max(err / A)) > 1e-5
