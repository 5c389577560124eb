"""The C ABI on the host: the library loads, exports what include/q2_0.h declares, and
rejects bad arguments with the documented status before touching the GPU.

No call here launches a kernel: every call either fails validation or is an empty
no-op, which returns before any HIP call, so these run without a GPU.
"""

import os
import re

import pytest

from ternary_bit_quantized_amd import q2_0 as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q2_0.h")

# Fake but aligned device addresses: validation never dereferences them.
P16, P4 = 1 << 20, (1 << 20) + 4


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(q2_0_[a-z0-9_]+)\s*\(", text))


def test_library_exports_every_declared_symbol():
    L = B.lib()
    declared = _declared()
    assert declared == set(B.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_version_and_status_strings():
    assert "gfx950" in B.version()
    for s in range(9):
        assert B.lib().q2_0_status_string(s).decode().startswith("Q2_0_")
    assert B.lib().q2_0_status_string(99) == b"unknown q2_0 status"
    assert B.lib().q2_0_last_hip_error() == 0


@pytest.mark.parametrize("K", [0, -64, 100, 63, 1 << 25])
def test_shape_errors(K):
    assert B.get_rows_raw(P16, 10, K, P4, 1, P16, max(K, 1)) == B.Q2_0_ERR_SHAPE
    assert B.mul_mat_vec_raw(P16, 10, K, P16, max(K, 1), 1, P16, 10) == B.Q2_0_ERR_SHAPE
    assert B.mul_mat_raw(P16, 10, K, P16, max(K, 1), 16, P16, 10, 0, 0, 0) == B.Q2_0_ERR_SHAPE


def test_negative_sizes():
    assert B.get_rows_raw(P16, -1, 64, P4, 1, P16, 64) == B.Q2_0_ERR_SHAPE
    assert B.get_rows_raw(P16, 1, 64, P4, -1, P16, 64) == B.Q2_0_ERR_SHAPE
    assert B.mul_mat_vec_raw(P16, 1, 64, P16, 64, -1, P16, 1) == B.Q2_0_ERR_SHAPE
    assert B.mul_mat_raw(P16, -5, 64, P16, 64, 16, P16, 1, 0, 0, 0) == B.Q2_0_ERR_SHAPE
    assert B.mul_mat_raw(P16, 5, 64, P16, 64, 65535 * 64 + 1, P16, 5, 0, 0, 0) == B.Q2_0_ERR_SHAPE


def test_empty_is_ok_even_with_null_pointers():
    assert B.get_rows_raw(0, 10, 64, 0, 0, 0, 64) == B.Q2_0_OK
    assert B.mul_mat_vec_raw(0, 0, 64, 0, 64, 1, 0, 0) == B.Q2_0_OK
    assert B.mul_mat_vec_raw(0, 10, 64, 0, 64, 0, 0, 10) == B.Q2_0_OK
    assert B.mul_mat_raw(0, 0, 64, 0, 64, 100, 0, 0, 0, 0, 0) == B.Q2_0_OK
    assert B.mul_mat_raw(0, 10, 64, 0, 64, 0, 0, 10, 1, 0, 0) == B.Q2_0_OK


def test_null_pointers():
    assert B.get_rows_raw(0, 10, 64, P4, 1, P16, 64) == B.Q2_0_ERR_NULL
    assert B.get_rows_raw(P16, 10, 64, 0, 1, P16, 64) == B.Q2_0_ERR_NULL
    assert B.get_rows_raw(P16, 10, 64, P4, 1, 0, 64) == B.Q2_0_ERR_NULL
    for args in [(0, P16, P16), (P16, 0, P16), (P16, P16, 0)]:
        w, x, y = args
        assert B.mul_mat_vec_raw(w, 10, 64, x, 64, 1, y, 10) == B.Q2_0_ERR_NULL
        assert B.mul_mat_raw(w, 10, 64, x, 64, 32, y, 10, 0, 0, 0) == B.Q2_0_ERR_NULL


def test_layout_errors():
    assert B.get_rows_raw(P16, 10, 128, P4, 1, P16, 127) == B.Q2_0_ERR_LAYOUT
    assert B.mul_mat_vec_raw(P16, 10, 128, P16, 127, 2, P16, 10) == B.Q2_0_ERR_LAYOUT
    assert B.mul_mat_vec_raw(P16, 10, 128, P16, 128, 2, P16, 9) == B.Q2_0_ERR_LAYOUT
    assert B.mul_mat_raw(P16, 10, 128, P16, 64, 20, P16, 10, 0, 0, 0) == B.Q2_0_ERR_LAYOUT


def test_alignment_errors():
    assert B.get_rows_raw(P16 + 1, 10, 64, P4, 1, P16, 64) == B.Q2_0_ERR_ALIGN
    assert B.get_rows_raw(P16, 10, 64, P4 + 2, 1, P16, 64) == B.Q2_0_ERR_ALIGN
    assert B.get_rows_raw(P16, 10, 64, P4, 1, P16 + 2, 64) == B.Q2_0_ERR_ALIGN
    assert B.mul_mat_vec_raw(P16 + 1, 10, 64, P16, 64, 1, P16, 10) == B.Q2_0_ERR_ALIGN
    assert B.mul_mat_vec_raw(P16, 10, 64, P16 + 2, 64, 1, P16, 10) == B.Q2_0_ERR_ALIGN
    assert B.mul_mat_raw(P16, 10, 64, P16, 64, 20, P16 + 1, 10, 0, 0, 0) == B.Q2_0_ERR_ALIGN


def test_unsupported():
    assert B.mul_mat_vec_raw(P16, 10, 64, P16, 64, 9, P16, 10) == B.Q2_0_ERR_UNSUPPORTED
    assert B.mul_mat_raw(P16, 10, 64, P16, 64, 20, P16, 10, 3, 0, 0) == B.Q2_0_ERR_UNSUPPORTED
    assert B.mul_mat_raw(P16, 10, 64, P16, 64, 20, P16, 10, -1, 0, 0) == B.Q2_0_ERR_UNSUPPORTED


def test_workspace_query_and_checks():
    # fp16 GEMM stages x as fp16: N*K*2 bytes and N int32 column exponents (each rounded
    # up to 256), plus split-K partials when the tile grid is small; nothing else needs any
    assert B.mul_mat_workspace_bytes(65536, 4096, 512, B.Q2_0_PREC_F16_MFMA) == 512 * 4096 * 2 + 2048
    assert B.mul_mat_workspace_bytes(65536, 4096, 100, B.Q2_0_PREC_F16_MFMA) == 100 * 4096 * 2 + 512
    assert B.mul_mat_workspace_bytes(1024, 4096, 512, B.Q2_0_PREC_F16_MFMA) > 512 * 4096 * 2
    assert B.mul_mat_workspace_bytes(4096, 4096, 512, B.Q2_0_PREC_F32) == 0
    assert B.mul_mat_workspace_bytes(4096, 4096, 8, B.Q2_0_PREC_F16_MFMA) == 0
    assert B.mul_mat_workspace_bytes(4096, 100, 512, B.Q2_0_PREC_F16_MFMA) == 0
    need = B.mul_mat_workspace_bytes(10, 64, 20, B.Q2_0_PREC_F16_MFMA)
    assert need >= 20 * 64 * 2
    assert B.mul_mat_raw(P16, 10, 64, P16, 64, 20, P16, 10, 0, P16, need - 1) == B.Q2_0_ERR_WORKSPACE
    assert B.mul_mat_raw(P16, 10, 64, P16, 64, 20, P16, 10, 0, 0, need) == B.Q2_0_ERR_WORKSPACE
    assert B.mul_mat_raw(P16, 10, 64, P16, 64, 20, P16, 10, 0, P16 + 8, need) == B.Q2_0_ERR_WORKSPACE
    # the fp32-grade matrix-core GEMM stages x as two fp16 halves; N <= 8 needs nothing
    F32M = B.Q2_0_PREC_F32_MFMA
    assert B.mul_mat_workspace_bytes(65536, 4096, 512, F32M) == 2 * 512 * 4096 * 2 + 2048
    assert B.mul_mat_workspace_bytes(4096, 4096, 8, F32M) == 0
    need = B.mul_mat_workspace_bytes(10, 64, 20, F32M)
    assert need >= 2 * 20 * 64 * 2
    assert B.mul_mat_raw(P16, 10, 64, P16, 64, 20, P16, 10, F32M, P16, need - 1) == B.Q2_0_ERR_WORKSPACE
    assert B.mul_mat_raw(P16, 10, 64, P16, 64, 20, P16, 10, F32M, 0, need) == B.Q2_0_ERR_WORKSPACE


def test_group_validation():
    items = B.make_items([(P16, 10, P16, 10), (P16, 5, P16 + 2, 5)])
    assert B.mul_mat_vec_group_raw(items, 2, 64, P16, 64, 1) == B.Q2_0_ERR_ALIGN
    assert B.mul_mat_vec_group_raw(items, 2, 100, P16, 100, 1) == B.Q2_0_ERR_SHAPE
    assert B.mul_mat_vec_group_raw(items, -1, 64, P16, 64, 1) == B.Q2_0_ERR_SHAPE
    assert B.mul_mat_vec_group_raw(None, 0, 64, P16, 64, 1) == B.Q2_0_OK
    assert B.mul_mat_vec_group_raw(None, 3, 64, P16, 64, 1) == B.Q2_0_ERR_NULL
    ok = B.make_items([(P16, 10, P16, 10), (0, 0, 0, 0)])
    assert B.mul_mat_vec_group_raw(ok, 2, 64, P16, 64, 9) == B.Q2_0_ERR_UNSUPPORTED
    assert B.mul_mat_vec_group_raw(ok, 2, 64, P16, 63, 1) == B.Q2_0_ERR_LAYOUT
    assert B.mul_mat_vec_group_raw(ok, 2, 64, 0, 64, 1) == B.Q2_0_ERR_NULL
    bad_ldy = B.make_items([(P16, 10, P16, 9)])
    assert B.mul_mat_vec_group_raw(bad_ldy, 1, 64, P16, 64, 1) == B.Q2_0_ERR_LAYOUT
    empty = B.make_items([(0, 0, 0, 0)])
    assert B.mul_mat_vec_group_raw(empty, 1, 64, 0, 64, 1) == B.Q2_0_OK


def test_gemm_group_validation_and_workspace():
    items = B.make_items([(P16, 10, P16, 10), (P16, 5, P16 + 2, 5)])
    assert B.mul_mat_group_raw(items, 2, 64, P16, 64, 20, 0, P16, 1 << 20) == B.Q2_0_ERR_ALIGN
    assert B.mul_mat_group_raw(items, 2, 100, P16, 100, 20, 0, P16, 1 << 20) == B.Q2_0_ERR_SHAPE
    assert B.mul_mat_group_raw(items, -1, 64, P16, 64, 20, 0, P16, 1 << 20) == B.Q2_0_ERR_SHAPE
    assert B.mul_mat_group_raw(None, 0, 64, P16, 64, 20, 0, 0, 0) == B.Q2_0_OK
    assert B.mul_mat_group_raw(None, 2, 64, P16, 64, 20, 0, 0, 0) == B.Q2_0_ERR_NULL
    ok = B.make_items([(P16, 10, P16, 10), (0, 0, 0, 0), (P16, 300, P16, 300)])
    assert B.mul_mat_group_raw(ok, 3, 64, P16, 64, 20, 7, P16, 1 << 20) == B.Q2_0_ERR_UNSUPPORTED
    assert B.mul_mat_group_raw(ok, 3, 64, P16, 63, 20, 0, P16, 1 << 20) == B.Q2_0_ERR_LAYOUT
    # workspace: x once for the whole group, split-K state for every item
    need = B.mul_mat_group_workspace_bytes(ok, 3, 64, 20, B.Q2_0_PREC_F16_MFMA)
    assert need >= 20 * 64 * 2
    assert B.mul_mat_group_raw(ok, 3, 64, P16, 64, 20, 0, P16, need - 1) == B.Q2_0_ERR_WORKSPACE
    assert B.mul_mat_group_raw(ok, 3, 64, P16, 64, 20, 0, 0, need) == B.Q2_0_ERR_WORKSPACE
    assert B.mul_mat_group_workspace_bytes(ok, 3, 64, 20, B.Q2_0_PREC_F32) == 0
    assert B.mul_mat_group_workspace_bytes(ok, 3, 64, 8, B.Q2_0_PREC_F16_MFMA) == 0
    big = B.make_items([(P16, 4096, P16, 4096), (P16, 1024, P16, 1024), (P16, 1024, P16, 1024)])
    g = B.mul_mat_group_workspace_bytes(big, 3, 4096, 512, B.Q2_0_PREC_F16_MFMA)
    singles = [B.mul_mat_workspace_bytes(M, 4096, 512, B.Q2_0_PREC_F16_MFMA) for M in (4096, 1024, 1024)]
    assert 512 * 4096 * 2 < g < sum(singles)   # x staged once, fewer splits than the small singles
    # the fp32-grade matrix-core precision: x as two fp16 halves for the group, nothing for N <= 8
    F32M = B.Q2_0_PREC_F32_MFMA
    need_m = B.mul_mat_group_workspace_bytes(ok, 3, 64, 20, F32M)
    assert need_m >= 2 * 20 * 64 * 2
    assert B.mul_mat_group_workspace_bytes(ok, 3, 64, 8, F32M) == 0
    assert B.mul_mat_group_raw(ok, 3, 64, P16, 64, 20, F32M, P16, need_m - 1) == B.Q2_0_ERR_WORKSPACE
    gm = B.mul_mat_group_workspace_bytes(big, 3, 4096, 512, F32M)
    assert gm >= 2 * 512 * 4096 * 2


def test_activation_type_validation():
    """The *_act entry points: an unknown activation type is UNSUPPORTED (checked before the
    alignment, which depends on it), 16-bit activations need 2-byte alignment only, and
    everything else is validated as for the F32 calls."""
    F16, BF16 = B.Q2_0_ACT_F16, B.Q2_0_ACT_BF16
    for bad in (-1, 3, 99):
        assert B.mul_mat_vec_act_raw(P16, 10, 64, P16 + 1, bad, 64, 1, P16, 10) == B.Q2_0_ERR_UNSUPPORTED
        assert B.mul_mat_act_raw(P16, 10, 64, P16, bad, 64, 20, P16, 10, 0, P16, 1 << 20) == B.Q2_0_ERR_UNSUPPORTED
    for xt in (F16, BF16):
        # a 2-byte offset is fine for 16-bit activations (passes validation), an odd address is not
        assert B.mul_mat_vec_act_raw(P16, 10, 64, P16 + 1, xt, 64, 1, P16, 10) == B.Q2_0_ERR_ALIGN
        assert B.mul_mat_act_raw(P16, 10, 64, P16 + 1, xt, 64, 20, P16, 10, 0, P16, 1 << 20) == B.Q2_0_ERR_ALIGN
        assert B.mul_mat_vec_act_raw(P16, 10, 64, P16 + 2, xt, 64, 9, P16, 10) == B.Q2_0_ERR_UNSUPPORTED
        assert B.mul_mat_vec_act_raw(P16, 10, 64, P16 + 2, xt, 63, 1, P16, 10) == B.Q2_0_ERR_LAYOUT
        assert B.mul_mat_vec_act_raw(P16, 10, 100, P16, xt, 100, 1, P16, 10) == B.Q2_0_ERR_SHAPE
        assert B.mul_mat_vec_act_raw(P16, 0, 64, 0, xt, 64, 1, 0, 0) == B.Q2_0_OK
        assert B.mul_mat_vec_act_raw(P16, 10, 64, 0, xt, 64, 1, P16, 10) == B.Q2_0_ERR_NULL
        need = B.mul_mat_workspace_bytes(10, 64, 20, B.Q2_0_PREC_F16_MFMA)
        assert B.mul_mat_act_raw(P16, 10, 64, P16 + 2, xt, 64, 20, P16, 10, 0, P16, need - 1) == B.Q2_0_ERR_WORKSPACE
        items = B.make_items([(P16, 10, P16, 10), (P16, 5, P16 + 2, 5)])
        assert B.mul_mat_vec_group_act_raw(items, 2, 64, P16 + 2, xt, 64, 1) == B.Q2_0_ERR_ALIGN   # y of item 1
        assert B.mul_mat_group_act_raw(items, 2, 64, P16 + 2, xt, 64, 20, 0, P16, 1 << 20) == B.Q2_0_ERR_ALIGN
        ok = B.make_items([(P16, 10, P16, 10)])
        assert B.mul_mat_vec_group_act_raw(ok, 1, 64, P16 + 1, xt, 64, 1) == B.Q2_0_ERR_ALIGN
        assert B.mul_mat_group_act_raw(ok, 1, 64, P16, 7, 64, 20, 0, P16, 1 << 20) == B.Q2_0_ERR_UNSUPPORTED
    # F32 through the *_act entry keeps the 4-byte rule
    assert B.mul_mat_vec_act_raw(P16, 10, 64, P16 + 2, B.Q2_0_ACT_F32, 64, 1, P16, 10) == B.Q2_0_ERR_ALIGN


def test_quantize_and_repack_validation():
    assert B.quantize_raw(P16, 10, 100, 100, P16) == B.Q2_0_ERR_SHAPE
    assert B.quantize_raw(P16, -1, 64, 64, P16) == B.Q2_0_ERR_SHAPE
    assert B.quantize_raw(0, 0, 64, 64, 0) == B.Q2_0_OK
    assert B.quantize_raw(0, 10, 64, 64, P16) == B.Q2_0_ERR_NULL
    assert B.quantize_raw(P16, 10, 64, 63, P16) == B.Q2_0_ERR_LAYOUT
    assert B.quantize_raw(P16 + 2, 10, 64, 64, P16) == B.Q2_0_ERR_ALIGN
    assert B.quantize_raw(P16, 10, 64, 64, P16 + 1) == B.Q2_0_ERR_ALIGN
    assert B.repack_g128_raw(P16, 10, 64, P16) == B.Q2_0_ERR_SHAPE      # K % 128 != 0
    assert B.repack_g128_raw(P16, 10, 100, P16) == B.Q2_0_ERR_SHAPE
    assert B.repack_g128_raw(0, 0, 128, 0) == B.Q2_0_OK
    assert B.repack_g128_raw(P16, 10, 128, 0) == B.Q2_0_ERR_NULL
    assert B.repack_g128_raw(P16 + 1, 10, 128, P16) == B.Q2_0_ERR_ALIGN


def test_mul_mat_id_validation():
    F16, F32 = B.Q2_0_PREC_F16_MFMA, B.Q2_0_PREC_F32
    ws = 1 << 24

    def call(w=P16, ne=4, M=10, K=64, x=P16, xt=B.Q2_0_ACT_F32, ldx=64, xs=1, ids=P16, nu=2, nt=3, y=P16, ldy=10,
             prec=F16, wsp=P16, wsb=ws):
        return B.mul_mat_id_raw(w, ne, M, K, x, xt, ldx, xs, ids, nu, nt, y, ldy, prec, wsp, wsb)

    assert call(K=100) == B.Q2_0_ERR_SHAPE
    assert call(ne=0) == B.Q2_0_ERR_SHAPE
    assert call(ne=8193) == B.Q2_0_ERR_SHAPE
    assert call(nu=1 << 11, nt=1 << 10) == B.Q2_0_ERR_SHAPE            # more than 2^20 pairs
    assert call(xs=3) == B.Q2_0_ERR_SHAPE                              # x_slots neither 1 nor n_used
    assert call(M=0, w=0, x=0, ids=0, y=0) == B.Q2_0_OK
    assert call(nt=0, w=0, x=0, ids=0, y=0) == B.Q2_0_OK
    assert call(ids=0) == B.Q2_0_ERR_NULL
    assert call(x=0) == B.Q2_0_ERR_NULL
    assert call(ldx=63) == B.Q2_0_ERR_LAYOUT
    assert call(ldy=9) == B.Q2_0_ERR_LAYOUT
    assert call(xt=5) == B.Q2_0_ERR_UNSUPPORTED
    assert call(ids=P16 + 2) == B.Q2_0_ERR_ALIGN
    assert call(x=P16 + 2) == B.Q2_0_ERR_ALIGN
    assert call(prec=3) == B.Q2_0_ERR_UNSUPPORTED
    # the fp32-grade matrix-core precision runs as Q2_0_PREC_F32 here (same workspace)
    assert (B.mul_mat_id_workspace_bytes(4, 10, 64, 2, 3, B.Q2_0_PREC_F32_MFMA) ==
            B.mul_mat_id_workspace_bytes(4, 10, 64, 2, 3, F32))
    need = B.mul_mat_id_workspace_bytes(4, 10, 64, 2, 3, F16)
    assert need >= 6 * 64 * 2 and B.mul_mat_id_workspace_bytes(4, 10, 64, 2, 3, F32) > 0
    assert call(wsb=need - 1) == B.Q2_0_ERR_WORKSPACE
    assert call(wsp=0) == B.Q2_0_ERR_WORKSPACE
    assert call(wsp=P16 + 8) == B.Q2_0_ERR_WORKSPACE
    assert B.mul_mat_id_workspace_bytes(0, 10, 64, 2, 3, F16) == 0


def test_mul_mat_noalloc_validation():
    """The allocation-free variant checks its arguments as q2_0_mul_mat does, then rejects
    calls whose scratch would exceed its static array -- all before any HIP call."""
    nr = B.mul_mat_noalloc_raw
    assert nr(P16, 10, 100, P16, 100, 16, P16, 10, 0) == B.Q2_0_ERR_SHAPE
    assert nr(0, 0, 64, 0, 64, 16, 0, 0, 0) == B.Q2_0_OK          # empty no-op
    assert nr(P16, 10, 64, 0, 64, 16, P16, 10, 0) == B.Q2_0_ERR_NULL
    assert nr(P16, 10, 64, P16, 63, 16, P16, 10, 0) == B.Q2_0_ERR_LAYOUT
    assert nr(P16 + 1, 10, 64, P16, 64, 16, P16, 10, 0) == B.Q2_0_ERR_ALIGN
    assert nr(P16, 10, 64, P16, 64, 16, P16, 10, 7) == B.Q2_0_ERR_UNSUPPORTED
    # 4096 x 12288 at N = 512 fits (46 MB, with its K split); at N = 4096 x alone is 100 MB
    assert 0 < B.mul_mat_workspace_bytes(4096, 12288, 512, 0) <= B.NOALLOC_SCRATCH_BYTES
    assert B.mul_mat_workspace_bytes(4096, 12288, 4096, 0) > B.NOALLOC_SCRATCH_BYTES
    assert nr(P16, 4096, 12288, P16, 12288, 4096, P16, 4096, 0) == B.Q2_0_ERR_TOO_LARGE
    assert B.lib().q2_0_status_string(B.Q2_0_ERR_TOO_LARGE).decode().startswith("Q2_0_ERR_TOO_LARGE")
    # the fp32-grade matrix-core precision stages x twice over: the limit comes at half the N
    F32M = B.Q2_0_PREC_F32_MFMA
    assert 0 < B.mul_mat_workspace_bytes(4096, 12288, 512, F32M) <= B.NOALLOC_SCRATCH_BYTES
    assert B.mul_mat_workspace_bytes(4096, 12288, 2048, F32M) > B.NOALLOC_SCRATCH_BYTES
    assert nr(P16, 4096, 12288, P16, 12288, 2048, P16, 4096, F32M) == B.Q2_0_ERR_TOO_LARGE


def test_mul_mat_vec_batch_validation():
    """Every item is checked before anything is launched; the call launches nothing on
    error or when it is empty."""
    mk = B.make_batch_items
    br = B.mul_mat_vec_batch_raw
    good = (P16, 10, 128, P16, 128, P16, 10)
    assert br(None, 0, 0, 1) == B.Q2_0_OK
    assert br(None, 2, 0, 1) == B.Q2_0_ERR_NULL
    assert br(mk([good]), -1, 0, 1) == B.Q2_0_ERR_SHAPE
    assert br(mk([good, (P16, 10, 100, P16, 128, P16, 10)]), 2, 0, 1) == B.Q2_0_ERR_SHAPE   # K % 64
    assert br(mk([good]), 1, 0, 0) == B.Q2_0_OK                                               # N = 0
    assert br(mk([(0, 0, 64, 0, 64, 0, 0)]), 1, 0, 1) == B.Q2_0_OK                            # M = 0 only
    assert br(mk([good, (P16, 10, 64, 0, 64, P16, 10)]), 2, 0, 1) == B.Q2_0_ERR_NULL
    assert br(mk([good, (P16, 10, 64, P16, 63, P16, 10)]), 2, 0, 1) == B.Q2_0_ERR_LAYOUT
    assert br(mk([good, (P16, 10, 64, P16, 64, P16, 9)]), 2, 0, 1) == B.Q2_0_ERR_LAYOUT
    assert br(mk([good]), 1, 7, 1) == B.Q2_0_ERR_UNSUPPORTED                                 # x_type
    assert br(mk([good, (P16 + 1, 10, 64, P16, 64, P16, 10)]), 2, 0, 1) == B.Q2_0_ERR_ALIGN
    assert br(mk([good]), 1, 0, 9) == B.Q2_0_ERR_UNSUPPORTED                                 # N > 8
