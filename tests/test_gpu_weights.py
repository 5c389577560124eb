"""GPU parity of the weight-side conversions: the reference quantizer (f32 -> Q2_0) and the
legacy group-128 reader, both bit for bit against the oracle."""

import numpy as np
import pytest

import oracle
from ternary_bit_quantized_amd import q2_0 as B
from ternary_bit_quantized_amd import synth

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def dev(a):
    return _torch().from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    _torch().cuda.synchronize()
    return t.cpu().numpy()


def gpu_quantize(wf, ld=None):
    torch = _torch()
    M, K = wf.shape
    ld = ld or K
    src = np.zeros((M, ld), dtype=np.float32)
    src[:, :K] = wf
    sd = dev(src)
    out = torch.full((M * (K // 64) * 18 + 7,), 0xAB, dtype=torch.uint8, device="cuda")
    st = B.quantize_raw(sd.data_ptr(), M, K, ld, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().q2_0_status_string(st)
    o = host(out)
    assert np.all(o[M * (K // 64) * 18:] == 0xAB), "wrote past the output"
    return o[:M * (K // 64) * 18].reshape(M, -1)


def weights_with_edge_blocks(seed, M, K):
    """Per-block magnitudes over 1e-9 .. 1e5 (scales that round to 0, fp16 subnormals,
    normals, and max|w| >= 65520, whose scale is inf), all-zero and signed-zero blocks,
    and blocks holding exact ties at +-d/2."""
    rng = np.random.default_rng(seed)
    nb = K // 64
    w = rng.standard_normal((M, nb, 64))
    w *= np.exp(rng.uniform(np.log(1e-9), np.log(1e5), size=(M, nb, 1)))
    w = w.astype(np.float32)
    flat = w.reshape(-1, 64)
    nblk = flat.shape[0]
    pick = rng.permutation(nblk)
    flat[pick[:nblk // 50]] = 0.0
    flat[pick[nblk // 50:nblk // 25]] = -0.0
    # ties: max |w| = d exactly (an fp16 value), other weights at +-d/2 and 0
    for b in pick[nblk // 25:nblk // 10]:
        d = np.float32(np.float16(rng.uniform(0.01, 100.0)))
        row = rng.choice(np.array([0.5, -0.5, 0.0, 0.25, -0.75], dtype=np.float32), size=64) * d
        row[rng.integers(0, 64)] = d if rng.random() < 0.5 else -d
        flat[b] = row
    return w.reshape(M, K)


@pytest.mark.parametrize("M,K,ld", [(1, 64, 64), (37, 640, 640), (300, 4096, 4096), (129, 1024, 1030)])
def test_quantize_matches_oracle_bitwise(M, K, ld):
    wf = weights_with_edge_blocks(M + K, M, K)
    got = gpu_quantize(wf, ld)
    ref = oracle.quantize_ref(wf)
    bad = np.flatnonzero((got != ref).any(axis=1))
    assert bad.size == 0, "rows %s differ (first block bytes %s vs %s)" % (bad[:5], got[bad[0]][:18], ref[bad[0]][:18])


def test_quantize_round_trips_ternary_weights():
    """Weights that are exactly d*t (t in {-1, 0, 1}, d an fp16 value, some t != 0 per block)
    come back bit for bit; all-zero blocks give d = 0 and code 1."""
    M, K = 513, 2048
    w = synth.weight(50, 0, 0, M, K, "tern", synth.ScaleDist("loguniform", 1e-3, 1e2, 0.02))
    dense = oracle.dequant(w, M, K).astype(np.float32)
    got = gpu_quantize(dense)
    # blocks with t == 0 everywhere carry no scale information: compare their codes only
    v = w.reshape(M, K // 64, 18)
    g = got.reshape(M, K // 64, 18)
    live = np.abs(dense.reshape(M, K // 64, 64)).max(axis=2) > 0
    assert np.array_equal(g[live], v[live])
    assert np.all(g[~live][:, :2] == 0) and np.all(g[~live][:, 2:] == 0x55)


def test_quantize_large_workload_shape():
    """A 12288 x 4096 matrix (the 8B gate projection): checked on sampled rows."""
    rng = np.random.default_rng(51)
    M, K = 12288, 4096
    wf = (rng.standard_normal((M, K)) * 0.02).astype(np.float32)
    got = gpu_quantize(wf)
    rows = np.unique(np.concatenate([rng.integers(0, M, 200), [0, M - 1]]))
    assert np.array_equal(got[rows], oracle.quantize_ref(wf[rows]))


@pytest.mark.parametrize("M,K", [(1, 128), (37, 640), (300, 4096)])
def test_repack_g128_matches_oracle_and_runs_through_the_mat_vec(M, K):
    torch = _torch()
    rng = np.random.default_rng(M + K)
    w128 = rng.integers(0, 256, size=(M, K // 128 * 34), dtype=np.uint8)
    # finite scales in [2^-8, 2) for the product check; the byte check covers any bytes
    w128v = w128.reshape(M, K // 128, 34)
    w128v[:, :, 1] &= 0x3F
    w128v[:, :, 1] |= 0x1C
    src = dev(w128)
    out = torch.full((M * (K // 64) * 18 + 5,), 0xCD, dtype=torch.uint8, device="cuda")
    st = B.repack_g128_raw(src.data_ptr(), M, K, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().q2_0_status_string(st)
    o = host(out)
    assert np.all(o[M * (K // 64) * 18:] == 0xCD)
    w64 = o[:M * (K // 64) * 18].reshape(M, -1)
    assert np.array_equal(w64, oracle.repack_g128(w128, M, K))
    # the repacked matrix multiplies like the legacy one (oracle decode of the legacy bytes)
    x = synth.activations(52, 0, 0, 2, K)
    yd = torch.empty((2, M), dtype=torch.float32, device="cuda")
    wd = dev(w64)
    xd = dev(x)
    st = B.mul_mat_vec_raw(wd.data_ptr(), M, K, xd.data_ptr(), K, 2, yd.data_ptr(), M,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    dense = oracle.dequant_g128(w128, M, K)
    y_ref = x.astype(np.float64) @ dense.T
    bound = np.abs(x.astype(np.float64)) @ np.abs(dense).T
    assert np.all(np.abs(host(yd) - y_ref) <= 1e-5 * bound)
