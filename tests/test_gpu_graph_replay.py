"""Calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed: every replay gives,
bit for bit, the eager call's result on the inputs the buffers hold at replay time.

The launches are the ones the benchmark times in graphs: the decode step's batch (one
8B layer's seven matrices, K = 4096 and K = 12288 segments, N = 1 in exact limbs and N = 2
in hi/lo halves), the prefill GEMM group with its planned K split, a split fp32-grade
GEMM, the no-allocation GEMM on its static scratch, the expert product at one token
(mat-vec pairs in K slices) and at 128 tokens (routing + routed GEMM), and get_rows.
Between replays the inputs are rewritten, the outputs poisoned with NaN, and unrelated
eager work and synchronizations run, so a replay that read stale inputs, skipped a
kernel, or depended on memory a previous call left behind would differ from the eager
result.  The eager results themselves are checked against the oracle by the parity
tests; here the reference is the same library called without a graph.
"""

import numpy as np
import pytest

from ternary_bit_quantized_amd import q2_0 as B
from ternary_bit_quantized_amd import synth

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _torch():
    import torch
    return torch


def dev(a):
    return _torch().from_numpy(np.ascontiguousarray(a)).cuda()


def bits(t):
    return t.detach().cpu().numpy().view(np.uint32).copy()


class Case:
    """Static input buffers (`inputs`), output buffers (`outputs`) and `run()`, which
    reads the first and writes the second with library calls only."""

    def __init__(self, inputs, outputs, run):
        self.inputs, self.outputs, self.run = inputs, outputs, run

    def load(self, values):
        for buf, v in zip(self.inputs, values):
            buf.copy_(v)

    def poison(self):
        for y in self.outputs:
            if y.dtype.is_floating_point:
                y.fill_(float("nan"))
            else:
                y.fill_(-1)


def eager_results(case, value_sets):
    torch = _torch()
    refs = []
    for vals in value_sets:
        case.load(vals)
        case.poison()
        case.run()
        torch.cuda.synchronize()
        refs.append([bits(y) for y in case.outputs])
    return refs


def unrelated_work(seed):
    torch = _torch()
    g = torch.Generator(device="cuda").manual_seed(seed)
    a = torch.randn(512, 512, device="cuda", generator=g)
    b = torch.randn(512, 512, device="cuda", generator=g)
    c = (a @ b).relu_().sum()
    torch.cuda.synchronize()
    return float(c)


def check_replays(case, value_sets, what):
    torch = _torch()
    refs = eager_results(case, value_sets)
    case.load(value_sets[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        case.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        case.run()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        i = (r + 1) % len(value_sets)        # start on the set the capture did not see last
        case.load(value_sets[i])
        case.poison()
        unrelated_work(100 + r)
        g.replay()
        torch.cuda.synchronize()
        for j, (y, ref) in enumerate(zip(case.outputs, refs[i])):
            got = bits(y)
            assert np.array_equal(got, ref), "%s: replay %d, output %d differs from the eager call (%d of %d)" % (
                what, r, j, int((got != ref).sum()), got.size)
        # eager call between replays on the same buffers, then a replay again
        case.run()
        torch.cuda.synchronize()
    del g


def value_sets(shapes, seed, n=2):
    """n sets of float32 activations of the given (rows, K) shapes."""
    out = []
    for s in range(n):
        out.append([_torch().from_numpy(synth.activations(seed, s, i, r, k)).cuda() for i, (r, k) in enumerate(shapes)])
    return out


_LAYER = {}


def layer_8b():
    if not _LAYER:
        wl = synth.STACK_8B
        _LAYER.update({n: (dev(synth.workload_weight(wl, n, 5)), wl.shapes[n]) for n in synth.MATS})
    return _LAYER


@pytest.mark.parametrize("N", [1, 2])
def test_decode_batch_replays(N):
    torch = _torch()
    mats = layer_8b()
    x4 = torch.empty((N, 4096), dtype=torch.float32, device="cuda")
    x12 = torch.empty((N, 12288), dtype=torch.float32, device="cuda")
    ys = [torch.empty((N, mats[n][1][0]), dtype=torch.float32, device="cuda") for n in synth.MATS]
    prods = [(mats[n][0], mats[n][1][0], mats[n][1][1], x12 if mats[n][1][1] == 12288 else x4) for n in synth.MATS]

    def run():
        B.q2_0_mul_mat_vec_batch(prods, ys=ys)

    check_replays(Case([x4, x12], ys, run), value_sets([(N, 4096), (N, 12288)], 71 + N, 3),
                  "decode batch N=%d" % N)


def test_mat_vec_group_replays():
    torch = _torch()
    mats = layer_8b()
    names = ("gate", "up")
    x = torch.empty((1, 4096), dtype=torch.float32, device="cuda")
    ys = [torch.empty((1, mats[n][1][0]), dtype=torch.float32, device="cuda") for n in names]

    def run():
        B.q2_0_mul_mat_vec_group([(mats[n][0], mats[n][1][0]) for n in names], 4096, x, ys=ys)

    check_replays(Case([x], ys, run), value_sets([(1, 4096)], 74), "mat-vec group gate/up")


@pytest.mark.parametrize("precision", [B.Q2_0_PREC_F16_MFMA, B.Q2_0_PREC_F32_MFMA])
def test_prefill_group_replays(precision):
    torch = _torch()
    mats = layer_8b()
    names = ("q", "k", "v")
    N, K = 512, 4096
    x = torch.empty((N, K), dtype=torch.float32, device="cuda")
    ys = [torch.empty((N, mats[n][1][0]), dtype=torch.float32, device="cuda") for n in names]
    items = B.make_items([(mats[n][0].data_ptr(), mats[n][1][0], y.data_ptr(), mats[n][1][0])
                          for n, y in zip(names, ys)])
    need = B.mul_mat_group_workspace_bytes(items, len(names), K, N, precision)
    wsp = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def run():
        B.q2_0_mul_mat_group([(mats[n][0], mats[n][1][0]) for n in names], K, x, precision, ys=ys, workspace=wsp)

    check_replays(Case([x], ys, run), value_sets([(N, K)], 75), "q/k/v group precision %d" % precision)


def test_split_k_gemm_and_noalloc_replays():
    """A call the planner splits in K (partials in the workspace), and the same product
    through the no-allocation entry point (partials in its static scratch), in one graph."""
    torch = _torch()
    M, K, N = 256, 12288, 16
    P = B.Q2_0_PREC_F32_MFMA
    w = dev(synth.weight(76, 0, 0, M, K, "quad", synth.ScaleDist("loguniform", 1e-3, 1e-1, 0.02)))
    x = torch.empty((N, K), dtype=torch.float32, device="cuda")
    y = torch.empty((N, M), dtype=torch.float32, device="cuda")
    y2 = torch.empty((N, M), dtype=torch.float32, device="cuda")
    need = B.mul_mat_workspace_bytes(M, K, N, P)
    wsp = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def run():
        B.q2_0_mul_mat(w, M, K, x, P, y=y, workspace=wsp)
        st = B.mul_mat_noalloc_raw(w.data_ptr(), M, K, x.data_ptr(), K, N, y2.data_ptr(), M, P,
                                   torch.cuda.current_stream().cuda_stream)
        assert st == 0, B.lib().q2_0_status_string(st)

    check_replays(Case([x], [y, y2], run), value_sets([(N, K)], 76), "split-K GEMM + noalloc")


@pytest.mark.parametrize("nt", [1, 128])
def test_expert_layer_replays(nt):
    """128 experts of 768 x 2048, 8 slots per token; the ids change between replays too."""
    from test_gpu_mul_mat_id import bench_experts
    torch = _torch()
    ne, M, K, nu = 128, 768, 2048, 8
    wall = dev(bench_experts())
    x = torch.empty((nt, K), dtype=torch.float32, device="cuda")
    ids = torch.empty((nt, nu), dtype=torch.int32, device="cuda")
    y = torch.empty((nt * nu, M), dtype=torch.float32, device="cuda")
    P = B.Q2_0_PREC_F16_MFMA
    need = B.mul_mat_id_workspace_bytes(ne, M, K, nu, nt, P)
    wsp = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

    def run():
        B.q2_0_mul_mat_id(wall, ne, M, K, x, ids, P, y=y, workspace=wsp)

    sets = []
    for s in range(3):
        rng = np.random.default_rng(77 + 10 * s + nt)
        idv = np.stack([rng.permutation(ne)[:nu] for _ in range(nt)]).astype(np.int32)
        sets.append([torch.from_numpy(synth.activations(77, s, nt, nt, K)).cuda(), torch.from_numpy(idv).cuda()])
    check_replays(Case([x, ids], [y], run), sets, "expert layer %d tokens" % nt)


def test_get_rows_replays():
    torch = _torch()
    mats = layer_8b()
    w, (M, K) = mats["q"]
    n = 2048
    ids = torch.empty(n, dtype=torch.int32, device="cuda")
    out = torch.empty((n, K), dtype=torch.float32, device="cuda")

    def run():
        B.q2_0_get_rows(w, M, K, ids, out=out)

    sets = [[torch.from_numpy(synth.row_ids(78, s, 0, n, M).astype(np.int32)).cuda()] for s in range(2)]
    check_replays(Case([ids], [out], run), sets, "get_rows 2048 of 4096")
