"""GPU parity of the 16-bit activation entry points (q2_0_*_act with Q2_0_ACT_F16 and
Q2_0_ACT_BF16) against the fp64 oracle, and their defining property: each element
enters the arithmetic as its exact f32 value, so the result equals, bit for bit, the
F32 call on the activations converted to f32.

Inputs are f32 draws rounded to half (numpy, nearest-even) or to bfloat16 (the input
helpers in synth, pinned against torch in the CPU suite); the oracle receives the exact
values of those 16-bit numbers.
"""

import numpy as np
import pytest

import oracle
from ternary_bit_quantized_amd import q2_0 as B
from ternary_bit_quantized_amd import synth

pytestmark = pytest.mark.gpu

REL_F32 = 1e-5
REL_F16 = 2e-3
TYPES = [B.Q2_0_ACT_F16, B.Q2_0_ACT_BF16]


def _torch():
    import torch
    return torch


def dev(a):
    return _torch().from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    _torch().cuda.synchronize()
    return t.cpu().numpy()


def act16(x, xt):
    """f32 draws -> (16-bit storage array (uint16/float16), exact f32 values)."""
    if xt == B.Q2_0_ACT_F16:
        h = synth.to_f16(x)
        return h, h.astype(np.float32)
    bits = synth.to_bf16_bits(x)
    return bits, synth.bf16_bits_to_f32(bits)


def padded(a, ld):
    out = np.zeros((a.shape[0], ld), dtype=a.dtype)
    out[:, :a.shape[1]] = a
    return out


def check(y, w, M, K, xv, rel, rows=None, what=""):
    y_ref, bound = oracle.mul_mat(w, M, K, xv, rows=rows)
    yy = y if rows is None else y[:, rows]
    r = oracle.check_products(yy, y_ref, bound, rel)
    assert r["ok"], "%s: %d/%d outside %.0e*bound, worst %.3g, first %s" % (
        what, r["n_bad"], r["n"], rel, r["max_err_over_bound"], r["first_bad"])


def mat_vec(w_d, M, K, x_store, xt, ldx, ldy=None):
    torch = _torch()
    N = x_store.shape[0]
    ldy = ldy or M
    xd = dev(padded(x_store, ldx))
    yd = torch.full((N, ldy), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    if xt is None:   # the F32 entry point
        st = B.mul_mat_vec_raw(w_d.data_ptr(), M, K, xd.data_ptr(), ldx, N, yd.data_ptr(), ldy, stream)
    else:
        st = B.mul_mat_vec_act_raw(w_d.data_ptr(), M, K, xd.data_ptr(), xt, ldx, N, yd.data_ptr(), ldy, stream)
    assert st == 0, B.lib().q2_0_status_string(st)
    y = host(yd)
    assert np.all(np.isnan(y[:, M:])), "wrote past M"
    return y[:, :M]


def mul_mat(w_d, M, K, x_store, xt, precision, ldx=None):
    torch = _torch()
    N = x_store.shape[0]
    ldx = ldx or K
    xd = dev(padded(x_store, ldx))
    yd = torch.full((N, M + 3), float("nan"), dtype=torch.float32, device="cuda")
    need = B.mul_mat_workspace_bytes(M, K, N, precision)
    wsd = torch.full((max(need, 16) // 4 + 1,), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    if xt is None:
        st = B.mul_mat_raw(w_d.data_ptr(), M, K, xd.data_ptr(), ldx, N, yd.data_ptr(), M + 3, precision,
                           wsd.data_ptr(), need, stream)
    else:
        st = B.mul_mat_act_raw(w_d.data_ptr(), M, K, xd.data_ptr(), xt, ldx, N, yd.data_ptr(), M + 3, precision,
                               wsd.data_ptr(), need, stream)
    assert st == 0, B.lib().q2_0_status_string(st)
    y = host(yd)
    assert np.all(np.isnan(y[:, M:])), "wrote past M"
    return y[:, :M]


# Mat-vec kernels: K-split (small M), streaming (M >= 16384 rows), generic (rows not
# 16-byte aligned: K/64 % 8 != 0, or x not aligned to four elements).
MV_CASES = [(300, 1024, 1, 1024), (300, 1024, 8, 1024), (2000, 4096, 3, 4100), (16400, 4096, 1, 4096),
            (16400, 4096, 4, 4096), (16384 + 7, 12288, 2, 12288), (77, 768, 5, 768), (300, 1024, 2, 1027)]


@pytest.mark.parametrize("xt", TYPES)
@pytest.mark.parametrize("M,K,N,ldx", MV_CASES)
def test_act_mat_vec_matches_oracle_and_f32_call(xt, M, K, N, ldx):
    w = synth.weight(40, M % 97, K // 64, M, K, "tern_c3", synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.01))
    xs, xv = act16(synth.activations(40, N, K // 64, N, K), xt)
    wd = dev(w)
    y = mat_vec(wd, M, K, xs, xt, ldx)
    rows = None if M * K * N <= 1 << 26 else np.unique(np.concatenate([np.arange(0, M, 11), [M - 1]]))
    check(y, w, M, K, xv, REL_F32, rows=rows, what="act %d mat-vec M=%d K=%d N=%d" % (xt, M, K, N))
    y32 = mat_vec(wd, M, K, xv, None, ldx)
    assert np.array_equal(y.view(np.uint32), y32.view(np.uint32)), "differs from the F32 call on the same values"


@pytest.mark.parametrize("xt", TYPES)
def test_act_mat_vec_value_range(xt):
    """Column magnitudes over the type's range (fp16: up to 65504 and into its subnormals;
    bf16: 1e-30 .. 1e30) and a 2^13 spread inside a column."""
    M, K, N = 16400, 4096, 4
    w = synth.weight(41, 0, 0, M, K, "tern_c3", synth.ScaleDist("uniform", 0.005, 0.05))
    x = synth.activations(41, 0, 1, N, K).astype(np.float64)
    mags = [6e4 / 8, 1e-4, 3.0, 1e-6] if xt == B.Q2_0_ACT_F16 else [1e30, 1e-30, 3.0, 1e8]
    x *= np.array(mags)[:, None]
    x[:, 1::2] *= 2.0 ** -13
    xs, xv = act16(x.astype(np.float32), xt)
    if xt == B.Q2_0_ACT_F16:
        assert np.isfinite(xv).all() and (np.abs(xv[3]) < 2.0 ** -14).any()   # subnormal halves present
    y = mat_vec(dev(w), M, K, xs, xt, K)
    check(y, w, M, K, xv, REL_F32, rows=np.arange(0, M, 13), what="act %d range" % xt)


@pytest.mark.parametrize("xt", TYPES)
@pytest.mark.parametrize("precision,rel", [(B.Q2_0_PREC_F16_MFMA, REL_F16), (B.Q2_0_PREC_F32, REL_F32)])
@pytest.mark.parametrize("M,K,N,ldx", [(300, 576, 130, 576), (1000, 4096, 96, 4098), (129, 12288, 18, 12288)])
def test_act_mul_mat_matches_oracle_and_f32_call(xt, precision, rel, M, K, N, ldx):
    w = synth.weight(42, N, K // 64, M, K, "quad", synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.02))
    xs, xv = act16(synth.activations(42, N, K // 64, N, K), xt)
    wd = dev(w)
    y = mul_mat(wd, M, K, xs, xt, precision, ldx)
    check(y, w, M, K, xv, rel, what="act %d GEMM p=%d M=%d K=%d N=%d" % (xt, precision, M, K, N))
    y32 = mul_mat(wd, M, K, xv, None, precision, ldx)
    assert np.array_equal(y.view(np.uint32), y32.view(np.uint32)), "differs from the F32 call on the same values"


@pytest.mark.parametrize("xt", TYPES)
def test_act_groups_match_oracle(xt):
    """Grouped mat-vec (N = 2) and grouped GEMM (N = 96, fp16 MFMA) with 16-bit activations."""
    torch = _torch()
    K = 4096
    Ms = (4096 // 4, 1024 // 4, 1024 // 4, 16384 + 3)
    mats = [(synth.weight(43, i, 0, M, K, "quad", synth.ScaleDist("uniform", 0.005, 0.05)), M)
            for i, M in enumerate(Ms)]
    stream = torch.cuda.current_stream().cuda_stream
    for N, rel in ((2, REL_F32), (96, REL_F16)):
        xs, xv = act16(synth.activations(43, N, 0, N, K), xt)
        xd = dev(xs)
        keep, entries, ys = [], [], []
        for w, M in mats:
            wd = dev(w)
            yd = torch.full((N, M + 3), float("nan"), dtype=torch.float32, device="cuda")
            keep.append(wd)
            ys.append(yd)
            entries.append((wd.data_ptr(), M, yd.data_ptr(), M + 3))
        items = B.make_items(entries)
        if N <= 8:
            st = B.mul_mat_vec_group_act_raw(items, len(entries), K, xd.data_ptr(), xt, K, N, stream)
        else:
            need = B.mul_mat_group_workspace_bytes(items, len(entries), K, N, B.Q2_0_PREC_F16_MFMA)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
            st = B.mul_mat_group_act_raw(items, len(entries), K, xd.data_ptr(), xt, K, N, B.Q2_0_PREC_F16_MFMA,
                                         ws.data_ptr(), need, stream)
        assert st == 0, B.lib().q2_0_status_string(st)
        for (w, M), yd in zip(mats, ys):
            y = host(yd)
            assert np.all(np.isnan(y[:, M:]))
            rows = np.unique(np.concatenate([np.arange(0, M, 7), [M - 1]]))
            check(y[:, :M], w, M, K, xv, rel, rows=rows, what="act %d group N=%d M=%d" % (xt, N, M))


def test_act_torch_wrappers_accept_half_and_bfloat16():
    torch = _torch()
    M, K = 300, 1024
    w = synth.weight(44, 0, 0, M, K, "quad", synth.ScaleDist("uniform", 0.005, 0.05))
    wd = dev(w)
    x32 = torch.from_numpy(synth.activations(44, 0, 0, 3, K)).cuda()
    for dt in (torch.float16, torch.bfloat16):
        x = x32.to(dt)
        y = B.q2_0_mul_mat_vec(wd, M, K, x)
        y_ref = B.q2_0_mul_mat_vec(wd, M, K, x.to(torch.float32))
        assert y.dtype == torch.float32 and torch.equal(y, y_ref)
        xb = torch.cat([x] * 40)   # N = 120: the GEMM
        g = B.q2_0_mul_mat(wd, M, K, xb)
        g_ref = B.q2_0_mul_mat(wd, M, K, xb.to(torch.float32))
        assert torch.equal(g, g_ref)
