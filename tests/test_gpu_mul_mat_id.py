"""GPU parity of the expert product q2_0_mul_mat_id against the oracle's definition (each
(token, slot) pair multiplied by its own expert), across routings: decode-like (one token,
eight experts), prefill-like (many tokens), every pair to one expert, unused experts,
out-of-range ids, both activation layouts, both precisions, 16-bit activations."""

import numpy as np
import pytest

import oracle
from ternary_bit_quantized_amd import q2_0 as B
from ternary_bit_quantized_amd import synth

pytestmark = pytest.mark.gpu

REL = {B.Q2_0_PREC_F16_MFMA: 2e-3, B.Q2_0_PREC_F32: 1e-5}


def _torch():
    import torch
    return torch


def dev(a):
    return _torch().from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    _torch().cuda.synchronize()
    return t.cpu().numpy()


def experts(seed, ne, M, K):
    return np.stack([synth.weight(seed, e, 0, M, K, "tern_c3", synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.01))
                     for e in range(ne)])


def run_id(wall, ne, M, K, x_store, xt, ids, precision, ldy=None, ldx=None):
    torch = _torch()
    nt, nu = ids.shape
    ldy = ldy or M
    ldx = ldx or K
    if ldx > K:                                    # strided x: each row padded to ldx elements
        pad = np.zeros((x_store.shape[0], ldx), dtype=x_store.dtype)
        pad[:, :K] = x_store
        x_store = pad
    wd, xd, idd = dev(wall), dev(x_store), dev(ids.astype(np.int32))
    x_slots = x_store.shape[0] // nt
    yd = torch.full((nt * nu, ldy), float("inf"), dtype=torch.float32, device="cuda")
    need = B.mul_mat_id_workspace_bytes(ne, M, K, nu, nt, precision)
    ws = torch.full((need // 4 + 1,), float("nan"), dtype=torch.float32, device="cuda")
    st = B.mul_mat_id_raw(wd.data_ptr(), ne, M, K, xd.data_ptr(), xt, ldx, x_slots, idd.data_ptr(), nu, nt,
                          yd.data_ptr(), ldy, precision, ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().q2_0_status_string(st)
    y = host(yd)
    assert np.all(np.isinf(y[:, M:])), "wrote past M"
    return y[:, :M]


def check(y, y_ref, bound, rel, what):
    bad = ~np.isfinite(y_ref)                      # out-of-range ids: NaN expected
    assert np.all(np.isnan(y[bad])), "%s: out-of-range pairs not NaN" % what
    r = oracle.check_products(np.where(bad, 0, y), np.where(bad, 0, y_ref), bound, rel)
    assert r["ok"], "%s: %d/%d outside %.0e*bound, worst %.3g, first %s" % (
        what, r["n_bad"], r["n"], rel, r["max_err_over_bound"], r["first_bad"])


# few pairs (<= 8 tokens, or fewer pairs than twice the experts) take one mat-vec per pair,
# more the expert-tiled GEMM
ROUTINGS = ["decode", "decode_bad_ids", "few_one_expert", "prefill", "one_expert", "bad_ids"]


def make_ids(kind, rng, ne):
    if kind == "decode":
        return rng.permutation(ne)[:8][None, :].astype(np.int32)          # 1 token, 8 distinct experts
    if kind == "decode_bad_ids":
        ids = rng.integers(0, ne, size=(4, 8)).astype(np.int32)
        ids[0, 2], ids[3, 7] = -5, ne
        return ids
    if kind == "few_one_expert":
        return np.full((8, 2), 5, dtype=np.int32)
    if kind == "prefill":
        return rng.integers(0, ne, size=(100, 8)).astype(np.int32)
    if kind == "one_expert":
        return np.full((150, 2), 3, dtype=np.int32)                       # 300 pairs, one expert
    ids = rng.integers(0, ne, size=(20, 4)).astype(np.int32)
    ids[3, 1], ids[7, 0], ids[19, 3] = -1, ne, 1 << 30
    return ids


@pytest.mark.parametrize("precision", [B.Q2_0_PREC_F16_MFMA, B.Q2_0_PREC_F32])
@pytest.mark.parametrize("kind", ROUTINGS)
@pytest.mark.parametrize("slots", ["token", "slot"])
def test_mul_mat_id_matches_oracle(precision, kind, slots):
    rng = np.random.default_rng(len(kind) * 7 + precision + len(slots))
    ne, M, K = 16, 300, 1024
    wall = experts(61, ne, M, K)
    ids = make_ids(kind, rng, ne)
    nt, nu = ids.shape
    rows = nt if slots == "token" else nt * nu
    x = synth.activations(61, rows, 0, rows, K)
    y = run_id(wall, ne, M, K, x, B.Q2_0_ACT_F32, ids, precision)
    y_ref, bound = oracle.mul_mat_id(wall, ne, M, K, x, ids)
    check(y, y_ref, bound, REL[precision], "%s/%s/p%d" % (kind, slots, precision))


@pytest.mark.parametrize("precision", [B.Q2_0_PREC_F16_MFMA, B.Q2_0_PREC_F32])
@pytest.mark.parametrize("ne", [511, 512, 600])
def test_mul_mat_id_many_experts(precision, ne):
    """Routing with 511 experts (the last count whose per-wave run counts fit in LDS), 512
    and 600 (the pair-by-pair placement): 300 tokens x 4 slots (two placement chunks),
    some ids out of range, every output checked."""
    rng = np.random.default_rng(ne + 10 * precision)
    M, K = 64, 128
    wall = experts(65, ne, M, K)
    ids = rng.integers(0, ne, size=(300, 4)).astype(np.int32)
    ids[5, 0], ids[77, 3], ids[299, 1] = -1, ne, ne + 1000
    x = synth.activations(65, 300, 0, 300, K)
    y = run_id(wall, ne, M, K, x, B.Q2_0_ACT_F32, ids, precision)
    y_ref, bound = oracle.mul_mat_id(wall, ne, M, K, x, ids)
    check(y, y_ref, bound, REL[precision], "ne=%d p%d" % (ne, precision))


@pytest.mark.parametrize("precision", [B.Q2_0_PREC_F16_MFMA, B.Q2_0_PREC_F32])
@pytest.mark.parametrize("ne,nt,nu", [(239, 512, 8), (240, 512, 8), (16, 513, 8)])
def test_mul_mat_id_routing_path_edges(precision, ne, nt, nu):
    """The edges of the one-pass routing (at most 4096 pairs and 240 runs: 239 experts at
    512 tokens x 8 slots) and of the chunk-by-chunk one it hands over to (240 experts:
    241 runs; 513 tokens: 4104 pairs); every output against the oracle, and bit for bit
    the same on a second call."""
    rng = np.random.default_rng(ne * 3 + nt + precision)
    M, K = 64, 128
    wall = experts(66, ne, M, K)
    ids = rng.integers(0, ne, size=(nt, nu)).astype(np.int32)
    ids[0, 0], ids[nt - 1, nu - 1] = -3, ne
    x = synth.activations(66, nt, 0, nt, K)
    y = run_id(wall, ne, M, K, x, B.Q2_0_ACT_F32, ids, precision)
    y2 = run_id(wall, ne, M, K, x, B.Q2_0_ACT_F32, ids, precision)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    y_ref, bound = oracle.mul_mat_id(wall, ne, M, K, x, ids)
    check(y, y_ref, bound, REL[precision], "ne=%d nt=%d p%d" % (ne, nt, precision))


@pytest.mark.parametrize("slots", ["token", "slot"])
@pytest.mark.parametrize("ne,nt", [(16, 60), (300, 160)])
def test_mul_mat_id_strided_x(slots, ne, nt):
    """x rows ldx = K + 1 elements apart (not a multiple of four: the conversion reads
    element by element), through the one-pass routing (16 experts) and the chunked one
    (300 experts; 640 pairs, enough to take the GEMM): bit for bit the result of the same x stored contiguously, and within
    the bound of the oracle."""
    rng = np.random.default_rng(ne + nt + len(slots))
    M, K, nu = 96, 512, 4
    wall = experts(67, ne, M, K)
    ids = rng.integers(0, ne, size=(nt, nu)).astype(np.int32)
    rows = nt if slots == "token" else nt * nu
    x = synth.activations(67, rows, 0, rows, K)
    p = B.Q2_0_PREC_F16_MFMA
    y = run_id(wall, ne, M, K, x, B.Q2_0_ACT_F32, ids, p, ldx=K + 1)
    y0 = run_id(wall, ne, M, K, x, B.Q2_0_ACT_F32, ids, p)
    assert np.array_equal(y.view(np.uint32), y0.view(np.uint32))
    y_ref, bound = oracle.mul_mat_id(wall, ne, M, K, x, ids)
    check(y, y_ref, bound, REL[p], "strided x ne=%d %s" % (ne, slots))


@pytest.mark.parametrize("precision", [B.Q2_0_PREC_F16_MFMA, B.Q2_0_PREC_F32])
def test_mul_mat_id_two_column_tiles_per_expert(precision):
    """256 experts with 65 pairs each: every expert's run spans two 64-column tiles, so the
    tile list is as long as it gets for this pair count and the fp16 path's scratch, laid
    out after it, must not overlap it; three ids out of range (NaN columns)."""
    rng = np.random.default_rng(257 + precision)
    ne, M, K, nu = 256, 96, 256, 5
    flat = rng.permutation(np.repeat(np.arange(ne, dtype=np.int32), 65))
    ids = flat.reshape(-1, nu).copy()
    ids[0, 0], ids[100, 4], ids[-1, 2] = -3, ne, ne + 7
    nt = ids.shape[0]
    wall = experts(67, ne, M, K)
    x = synth.activations(67, nt, 0, nt, K)
    y = run_id(wall, ne, M, K, x, B.Q2_0_ACT_F32, ids, precision)
    y_ref, bound = oracle.mul_mat_id(wall, ne, M, K, x, ids)
    check(y, y_ref, bound, REL[precision], "two tiles p%d" % precision)


def test_mul_mat_id_f32_equals_per_expert_mul_mat_bitwise():
    """On the fp32 path each result column depends only on its expert and activation, so it
    equals, bit for bit, q2_0_mul_mat of that expert on the gathered columns."""
    torch = _torch()
    rng = np.random.default_rng(62)
    ne, M, K = 8, 257, 2048
    wall = experts(62, ne, M, K)
    ids = rng.integers(0, ne, size=(40, 4)).astype(np.int32)
    x = synth.activations(62, 0, 0, 40, K)
    y = run_id(wall, ne, M, K, x, B.Q2_0_ACT_F32, ids, B.Q2_0_PREC_F32)
    flat = ids.reshape(-1)
    for e in range(ne):
        sel = np.flatnonzero(flat == e)
        if sel.size <= 8:          # q2_0_mul_mat sends N <= 8 to the mat-vec: another kernel
            continue
        xe = x[sel // 4]
        ye = B.q2_0_mul_mat(dev(wall[e]), M, K, dev(xe), precision=B.Q2_0_PREC_F32)
        assert np.array_equal(host(ye).view(np.uint32), y[sel].view(np.uint32)), "expert %d" % e


def test_mul_mat_id_large_expert_layer_and_determinism():
    """An expert layer of 64 experts shaped like a gate projection (768 x 2048), 512
    tokens x 8 slots, f16 activations; sampled pairs against the oracle; two calls agree
    bit for bit."""
    rng = np.random.default_rng(63)
    ne, M, K, nt, nu = 64, 768, 2048, 512, 8
    wall = experts(63, ne, M, K)
    ids = np.stack([rng.permutation(ne)[:nu] for _ in range(nt)]).astype(np.int32)
    xs = synth.to_f16(synth.activations(63, 0, 0, nt, K))
    y1 = run_id(wall, ne, M, K, xs, B.Q2_0_ACT_F16, ids, B.Q2_0_PREC_F16_MFMA)
    y2 = run_id(wall, ne, M, K, xs, B.Q2_0_ACT_F16, ids, B.Q2_0_PREC_F16_MFMA)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    pick = rng.choice(nt, size=12, replace=False)
    sub_ids = ids[pick]
    y_ref, bound = oracle.mul_mat_id(wall, ne, M, K, xs[pick].astype(np.float32), sub_ids)
    rows = (pick[:, None] * nu + np.arange(nu)[None, :]).reshape(-1)
    check(y1[rows], y_ref, bound, REL[B.Q2_0_PREC_F16_MFMA], "large layer")


def test_mul_mat_id_torch_wrapper():
    torch = _torch()
    ne, M, K = 4, 130, 512
    wall = experts(64, ne, M, K)
    ids = torch.tensor([[0, 3], [2, 2], [1, 0]], dtype=torch.int32, device="cuda")
    x = torch.from_numpy(synth.activations(64, 0, 0, 3, K)).cuda()
    y = B.q2_0_mul_mat_id(dev(wall), ne, M, K, x, ids, precision=B.Q2_0_PREC_F32)
    y_ref, bound = oracle.mul_mat_id(wall, ne, M, K, x.cpu().numpy(), ids.cpu().numpy())
    check(host(y), y_ref, bound, 1e-5, "wrapper")


_BENCH_EXPERTS = {}


def bench_experts():
    """128 experts of 768 x 2048, the expert layer the benchmark times."""
    if "w" not in _BENCH_EXPERTS:
        _BENCH_EXPERTS["w"] = experts(65, 128, 768, 2048)
    return _BENCH_EXPERTS["w"]


@pytest.mark.parametrize("nt,nu", [(1, 8), (1, 2), (3, 8), (16, 8), (128, 8), (512, 8)])
def test_mul_mat_id_bench_expert_layer(nt, nu):
    """The benchmark's expert layer (128 experts of 768 x 2048) at its token counts, on the
    fast precision: one fp32-grade mat-vec per pair up to 8 tokens and while the pairs are
    fewer than twice the experts (1 token x 8 slots: K in 2 slices; 1 x 2: in 4; 3 x 8: in
    1; 16 x 8), more pairs the routed fp16 GEMM.  Sampled tokens against the oracle, each at
    the tolerance of the path that served it."""
    ne, M, K = 128, 768, 2048
    rng = np.random.default_rng(65 + nt * 10 + nu)
    wall = bench_experts()
    ids = np.stack([rng.permutation(ne)[:nu] for _ in range(nt)]).astype(np.int32)
    x = synth.activations(65, nt, nu, nt, K)
    y = run_id(wall, ne, M, K, x, B.Q2_0_ACT_F32, ids, B.Q2_0_PREC_F16_MFMA)
    pick = np.sort(rng.choice(nt, size=min(nt, 12), replace=False))
    y_ref, bound = oracle.mul_mat_id(wall, ne, M, K, x[pick], ids[pick])
    rows = (pick[:, None] * nu + np.arange(nu)[None, :]).reshape(-1)
    per_pair = nt <= 8 or nt * nu < 2 * ne
    rel = REL[B.Q2_0_PREC_F32] if per_pair else REL[B.Q2_0_PREC_F16_MFMA]
    check(y[rows], y_ref, bound, rel, "bench layer nt=%d nu=%d" % (nt, nu))


@pytest.mark.parametrize("nt,nu,ne", [(24, 8, 128), (31, 8, 128), (32, 8, 128), (40, 4, 96)])
def test_mul_mat_id_few_pairs_per_expert(nt, nu, ne):
    """More than 8 tokens but fewer pairs than twice the experts (24 and 31 tokens x 8 slots
    over 128 experts, and 40 x 4 over 96) take the per-pair mat-vec on the fast precision;
    32 x 8 = 256 pairs (exactly twice) takes the GEMM.  A few ids out of range give NaN
    columns.  Every output against the oracle at the tolerance of the path that served it."""
    M, K = 200, 1024
    rng = np.random.default_rng(nt * 100 + nu + ne)
    wall = experts(71, ne, M, K)
    ids = rng.integers(0, ne, size=(nt, nu)).astype(np.int32)
    ids[1, 0], ids[nt - 1, nu - 1] = -3, ne
    x = synth.activations(71, nt, nu, nt, K)
    y = run_id(wall, ne, M, K, x, B.Q2_0_ACT_F32, ids, B.Q2_0_PREC_F16_MFMA)
    y_ref, bound = oracle.mul_mat_id(wall, ne, M, K, x, ids)
    per_pair = nt * nu < 2 * ne
    rel = REL[B.Q2_0_PREC_F32] if per_pair else REL[B.Q2_0_PREC_F16_MFMA]
    check(y, y_ref, bound, rel, "few pairs nt=%d nu=%d ne=%d" % (nt, nu, ne))
