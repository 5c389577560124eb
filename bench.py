"""Benchmark of the Q2_0 hot path on one MI355X.

Workload: a Qwen3-8B-shaped ternary model's linear work -- the 36-layer stack of
q/o 4096x4096, k/v 1024x4096, gate/up 12288x4096 and down 4096x12288 Q2_0 matrices
(1.95 GB) plus a 151936x4096 Q2_0 vocabulary tensor used both as the embedding
(get_rows) and as the LM head -- with seeded synthetic weights and activations.  Each
matrix kind is stored as one tensor of its 36 layers (layer l's q is rows l*4096 ..),
so a layer's matrix is a view and all layers' q projections are one taller matrix.

One step is one pass of the whole hot path:
  prefill: get_rows of 512 token ids, then the 252 stack matrices at N = 512 on the
           fp16-MFMA GEMM, per layer as the model runs them: q/k/v as one group call
           (they share the input), o, gate/up as one group call, down;
  decode : get_rows of 1 token id, then the 252 stack matrices and the LM head at
           N = 1 on the mat-vec, in one batched launch: the workload uses one
           activation per distinct K, so the launch has two activation segments (the
           K = 4096 matrices with the head, and the K = 12288 down projections).
The prefill parts are captured once in HIP graphs and replayed; the decode parts are
single launches and go out directly, behind the prefill on the same stream (a graph
replay of one launch would add its own ~20 us; that figure is reported beside).  Inputs
are resident in HBM before timing starts.

`value` is that decode launch's stream rate in GB/s (algorithmic bytes: Q2_0 weights +
f32 activations + f32 outputs, over its time): a property of the kernel, which can
batch matrices of different layers because this workload's activations do not depend
on each other.  A transformer cannot: each layer's input comes from the layer before.
The decode is therefore also timed under the schedule such a model runs -- per layer,
q/k/v as one group call, o, gate/up as one call, down (144 launches + the head) -- and
`decode_tokens_per_s` comes from that schedule; the one-launch figure is reported as
`decode_tokens_per_s_kernel_stream_bound`.

Measured beside the step (not part of it): the other workloads of the configuration
list (the Qwen3-1.7B-shaped decode on a rotation of 56 layer copies at N = 1 and 8,
its prefill at N = 512, the vocabulary tensor's get_rows and LM head on 4 rotated
copies, the tiny case), the widened rows (16-bit activations, the quantizer, the
group-128 reader, an expert layer), ceilings measured with this repository's own
kernels (HBM read stream, register-only MFMA loop, empty launch), and the CPU oracle on
a bounded sample.

Profiling: --eager launches the selected --parts directly (no graphs), and
--copy-calibration-mib runs one elementwise copy-like kernel (torch.neg) of known
size first, whose counter readings scale the kernels' FETCH_SIZE / WRITE_SIZE to
bytes.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q2_0 mat-vec GB/s (% HBM peak) at N=1; prefill GEMM TFLOP/s; tokens/s"
HBM_PEAK_GBS = 8000.0
F16_MFMA_PEAK_TFLOPS = 2500.0
PREFILL_N = 512

DECODE_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "mat_vec_bcast_qwen3_8b_decode_hbm_traffic.md")
GEMM_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemm_f16_qwen3_8b_prefill_hbm_traffic.md")
MFMA_PROFILE = os.path.join(ROOT, "profiles", "gemm_f16_qwen3_8b_prefill_mfma_utilisation.md")
CEIL_LIB = os.path.join(ROOT, "ternary_bit_quantized_amd", "libq2_0_ceilings.so")


def kernel_sources_sha256(names) -> str:
    """sha256 over the code of the named sources in csrc/ (in the order given; comments and
    blank lines removed, so that a comment edit keeps it), to tell whether recorded counter
    readings still describe the kernels being timed."""
    import hashlib
    import re
    h = hashlib.sha256()
    src = os.path.join(ROOT, "ternary_bit_quantized_amd", "csrc")
    for name in names:
        with open(os.path.join(src, name), encoding="utf-8") as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        code = "\n".join(ln.rstrip() for ln in (re.sub(r"//.*", "", l) for l in text.splitlines()) if ln.strip())
        h.update(name.encode() + b"\0" + code.encode())
    return h.hexdigest()


def recorded(path: str, prefix: str) -> dict:
    """`<prefix> <key>: <number>` lines of a committed profile summary, or {} when the
    sources it names (line `sources: a.hip, b.h`) changed after it was taken (line
    `sources_sha256: <hex>`)."""
    try:
        with open(path) as f:
            lines = f.read().splitlines()
    except OSError:
        return {}
    out, sha, names = {}, None, None
    for ln in lines:
        ln = ln.strip().strip("`")
        if ln.startswith("sources_sha256:"):
            sha = ln.split(":", 1)[1].strip()
        elif ln.startswith("sources:"):
            names = [n.strip() for n in ln.split(":", 1)[1].split(",") if n.strip()]
        elif ln.startswith(prefix + " "):
            key, val = ln[len(prefix) + 1:].split(":", 1)
            out[key.strip()] = float(val)
    try:
        ok = bool(names) and sha == kernel_sources_sha256(names)
    except OSError:
        ok = False
    return out if ok else {}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=36, help="stack layers (36 = the full model)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the other workloads and the ceilings")
    p.add_argument("--cpu-prefill-row-stride", type=int, default=16)
    p.add_argument("--cpu-decode-repeats", type=int, default=8)
    p.add_argument("--eager", action="store_true", help="launch parts directly, without HIP graphs")
    p.add_argument("--parts", default="", help="comma-separated subset of parts to run (profiling)")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="one device-to-device copy of this size before the parts (counter scaling)")
    return p.parse_args()


def mat_bytes(M, K, N):
    return M * (K // 64) * 18 + 4 * K * N + 4 * M * N


def graph_ms(torch, fn, reps):
    """fn captured once in a HIP graph; mean ms per replay over reps replays (HIP events on
    the replay stream), after two warm-up replays."""
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


class Stack:
    """A model's linear layers on the GPU, one tensor per matrix kind holding all layers."""

    def __init__(self, torch, dev, wl, layers, synth):
        self.wl, self.L = wl, layers
        host = synth.stack_weights(wl, range(layers), threads=min(16, os.cpu_count() or 8))
        self.host = host
        self.W = {}
        for n, (M, K) in wl.shapes.items():
            t = torch.empty((layers * M, K // 64 * 18), dtype=torch.uint8, device=dev)
            for l in range(layers):
                t[l * M:(l + 1) * M].copy_(torch.from_numpy(host[(l, n)]))
            self.W[n] = t

    def w(self, l, n):
        M = self.wl.shapes[n][0]
        return self.W[n][l * M:(l + 1) * M]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from ternary_bit_quantized_amd import q2_0 as B
    from ternary_bit_quantized_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    B.lib()

    wl, vwl = synth.STACK_8B, synth.VOCAB_8B
    L = args.layers
    t0 = time.time()
    stk = Stack(torch, dev, wl, L, synth)
    emb_host = synth.workload_weight(vwl, "emb")
    emb = torch.from_numpy(emb_host).to(dev)
    log("generated and uploaded %d matrices + vocab tensor in %.1f s" % (7 * L, time.time() - t0))

    VM, VK = vwl.shapes["emb"]
    Ks = sorted({K for (_, K) in wl.shapes.values()})
    x1 = {K: torch.from_numpy(synth.activations(wl.seed, 0, synth.stack_x_matrix_index(K), 1, K)).to(dev)
          for K in Ks}
    xP = {K: torch.from_numpy(synth.activations(wl.seed, 1, synth.stack_x_matrix_index(K), PREFILL_N, K)).to(dev)
          for K in Ks}
    ids_p = torch.from_numpy(synth.row_ids(vwl.seed, 0, 0, PREFILL_N, VM)).to(dev)
    ids_d = torch.from_numpy(synth.row_ids(vwl.seed, 1, 0, 1, VM)).to(dev)
    emb_out_p = torch.empty((PREFILL_N, VK), dtype=torch.float32, device=dev)
    emb_out_d = torch.empty((1, VK), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("inputs resident on the GPU")

    order = [(l, n) for l in range(L) for n in synth.MATS]

    def check(st, what):
        if st != 0:
            raise RuntimeError("%s failed: %s" % (what, B.lib().q2_0_status_string(st).decode()))

    def s():
        return torch.cuda.current_stream().cuda_stream

    def run_get_rows(ids, out):
        check(B.get_rows_raw(emb.data_ptr(), VM, VK, ids.data_ptr(), ids.numel(), out.data_ptr(), VK, s()),
              "get_rows")

    # decode outputs: one buffer per matrix kind (all layers), and the head's
    yst = {n: torch.empty((1, L * M), dtype=torch.float32, device=dev) for n, (M, K) in wl.shapes.items()}
    yh = torch.empty((1, VM), dtype=torch.float32, device=dev)

    def head(st):
        check(B.mul_mat_vec_raw(emb.data_ptr(), VM, VK, x1[VK].data_ptr(), VK, 1, yh.data_ptr(), VM, st),
              "lm_head")

    # the step's decode: every matrix of the token and the head in one batched launch
    def batch_items(xs):
        ent = []
        for n in ("q", "k", "v", "o", "gate", "up", "down"):
            M, K = wl.shapes[n]
            ent.append((stk.W[n].data_ptr(), L * M, K, xs[K].data_ptr(), K, yst[n].data_ptr(), L * M))
            if n == "up":   # the head reads the K = 4096 activation: same segment
                ent.append((emb.data_ptr(), VM, VK, xs[VK].data_ptr(), VK, yh.data_ptr(), VM))
        return B.make_batch_items(ent), len(ent)
    dec_items, n_dec_items = batch_items(x1)

    def run_decode_matvecs():
        check(B.mul_mat_vec_batch_raw(dec_items, n_dec_items, B.Q2_0_ACT_F32, 1, s()), "mat_vec_batch")

    # the schedule a transformer runs: per layer q/k/v, o, gate/up, down, then the head
    def ypl(l, n):
        M = wl.shapes[n][0]
        return yst[n][:, l * M:(l + 1) * M]

    layer_groups = []
    for l in range(L):
        for names in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
            it = B.make_items([(stk.w(l, n).data_ptr(), wl.shapes[n][0], ypl(l, n).data_ptr(), wl.shapes[n][0])
                               for n in names])
            layer_groups.append((it, len(names), wl.shapes[names[0]][1]))

    def run_decode_per_layer():
        st = s()
        for items, n, K in layer_groups:
            check(B.mul_mat_vec_group_raw(items, n, K, x1[K].data_ptr(), K, 1, st), "mat_vec_group")
        head(st)

    def run_decode_per_matrix():
        st = s()
        for l, n in order:
            M, K = wl.shapes[n]
            check(B.mul_mat_vec_raw(stk.w(l, n).data_ptr(), M, K, x1[K].data_ptr(), K, 1, ypl(l, n).data_ptr(),
                                    M, st), "mat_vec")
        head(st)

    # prefill: one output buffer per matrix kind; a layer's matrices that share x run as a group
    yPn = {n: torch.empty((PREFILL_N, wl.shapes[n][0]), dtype=torch.float32, device=dev) for n in synth.MATS}
    prefill_names = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))

    def prefill_items(l, names):
        return B.make_items([(stk.w(l, n).data_ptr(), wl.shapes[n][0], yPn[n].data_ptr(), wl.shapes[n][0])
                             for n in names])

    prefill_groups = [(prefill_items(l, names), len(names), wl.shapes[names[0]][1])
                      for l in range(L) for names in prefill_names]
    ws_bytes = max(max(B.mul_mat_group_workspace_bytes(items, n, K, PREFILL_N, p_)
                       for (items, n, K) in prefill_groups for p_ in (B.Q2_0_PREC_F16_MFMA, B.Q2_0_PREC_F32_MFMA)),
                   max(B.mul_mat_workspace_bytes(M, K, PREFILL_N, B.Q2_0_PREC_F16_MFMA)
                       for (M, K) in wl.shapes.values()))
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def run_prefill_gemms(precision=B.Q2_0_PREC_F16_MFMA, groups=None, xs=None, xt=B.Q2_0_ACT_F32):
        st = s()
        xs = xs or xP
        for items, n, K in (groups or prefill_groups):
            check(B.mul_mat_group_act_raw(items, n, K, xs[K].data_ptr(), xt, K, PREFILL_N, precision,
                                          ws.data_ptr(), ws_bytes, st), "mul_mat_group")

    def run_prefill_per_matrix():
        st = s()
        for l, n in order:
            M, K = wl.shapes[n]
            check(B.mul_mat_raw(stk.w(l, n).data_ptr(), M, K, xP[K].data_ptr(), K, PREFILL_N,
                                yPn[n].data_ptr(), M, B.Q2_0_PREC_F16_MFMA, ws.data_ptr(), ws_bytes, st),
                  "mul_mat")

    # ---- the widened rows, measured beside the step (not part of it): 16-bit activations,
    # the quantizer and the legacy group-128 reader, an expert layer
    x1h = {K: v.to(torch.float16) for K, v in x1.items()}
    xPb = {K: v.to(torch.bfloat16) for K, v in xP.items()}
    dec_items_h, _ = batch_items(x1h)

    def run_decode_f16_activations():
        check(B.mul_mat_vec_batch_raw(dec_items_h, n_dec_items, B.Q2_0_ACT_F16, 1, s()), "mat_vec_batch f16")

    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    qsrc = torch.randn((VM, VK), generator=gen, device=dev) * 0.02      # the vocabulary tensor's shape in f32
    qdst = torch.empty_like(emb)
    g128_src = emb.view(-1)[:VM * (VK // 128) * 34]                     # any bytes: a legacy-layout stand-in

    def run_quantize():
        check(B.quantize_raw(qsrc.data_ptr(), VM, VK, VK, qdst.data_ptr(), s()), "quantize")

    def run_repack_g128():
        check(B.repack_g128_raw(g128_src.data_ptr(), VM, VK, qdst.data_ptr(), s()), "repack_g128")

    # an expert layer: 128 experts of 768 x 2048 (random blocks with finite scales), 8 of
    # them per token; prefill 512 tokens on the fp16 GEMM, decode one token on the mat-vec
    MOE_E, MOE_M, MOE_K, MOE_USED = 128, 768, 2048, 8
    MOE_CALLS = 20
    moe_w = torch.randint(0, 256, (MOE_E * MOE_M, MOE_K // 64, 18), dtype=torch.uint8, device=dev, generator=gen)
    moe_w[:, :, 1] &= 0x3B
    moe_ids_p = torch.stack([torch.randperm(MOE_E, device=dev, generator=gen)[:MOE_USED]
                             for _ in range(PREFILL_N)]).to(torch.int32)
    moe_ids_d = moe_ids_p[:1].contiguous()
    moe_x = torch.randn((PREFILL_N, MOE_K), generator=gen, device=dev)
    moe_y = torch.empty((PREFILL_N * MOE_USED, MOE_M), dtype=torch.float32, device=dev)
    moe_ws_bytes = max(B.mul_mat_id_workspace_bytes(MOE_E, MOE_M, MOE_K, MOE_USED, PREFILL_N, p_)
                       for p_ in (B.Q2_0_PREC_F16_MFMA, B.Q2_0_PREC_F32))
    moe_ws = torch.empty(moe_ws_bytes, dtype=torch.uint8, device=dev)

    def run_moe(ids, precision):
        nt = ids.shape[0]
        check(B.mul_mat_id_raw(moe_w.data_ptr(), MOE_E, MOE_M, MOE_K, moe_x.data_ptr(), B.Q2_0_ACT_F32, MOE_K, 1,
                               ids.data_ptr(), MOE_USED, nt, moe_y.data_ptr(), MOE_M, precision,
                               moe_ws.data_ptr(), moe_ws_bytes, s()), "mul_mat_id")

    # ---- the parts
    parts = {
        "prefill_get_rows": lambda: run_get_rows(ids_p, emb_out_p),
        "prefill_gemm": run_prefill_gemms,
        "decode_get_rows": lambda: run_get_rows(ids_d, emb_out_d),
        "decode_mat_vec": run_decode_matvecs,
        "decode_mat_vec_per_layer": run_decode_per_layer,
        "decode_mat_vec_per_matrix": run_decode_per_matrix,
        "prefill_gemm_per_matrix": run_prefill_per_matrix,
        "prefill_gemm_f32_layer0": lambda: run_prefill_gemms(B.Q2_0_PREC_F32, groups=prefill_groups[:4]),
        "prefill_gemm_f32_mfma": lambda: run_prefill_gemms(B.Q2_0_PREC_F32_MFMA),
        "decode_mat_vec_f16_activations": run_decode_f16_activations,
        "prefill_gemm_bf16_activations": lambda: run_prefill_gemms(xs=xPb, xt=B.Q2_0_ACT_BF16),
        "quantize_vocab_f32": run_quantize,
        "repack_g128_vocab": run_repack_g128,
        "expert_layer_prefill": lambda: run_moe(moe_ids_p, B.Q2_0_PREC_F16_MFMA),
        "expert_layer_decode": lambda: run_moe(moe_ids_d, B.Q2_0_PREC_F16_MFMA),
    }
    if args.parts:
        keep = args.parts.split(",")
        parts = {k: v for k, v in parts.items() if k in keep}
    if args.copy_calibration_mib:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)      # one elementwise kernel: reads and writes nbytes each
        torch.cuda.synchronize()
        log("calibration kernel over %d bytes done" % nbytes)
        del src, dst
    if args.eager:
        for name, fn in parts.items():
            fn()
        torch.cuda.synchronize()
        log("eager parts done: %s" % ",".join(parts))
        return
    graphs = {}
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for name, fn in parts.items():   # eager warm-up on the capture stream
            fn()
    torch.cuda.synchronize()
    for name, fn in parts.items():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs[name] = g
    torch.cuda.synchronize()
    log("graphs captured")

    step_parts = [p for p in ("prefill_get_rows", "prefill_gemm", "decode_get_rows", "decode_mat_vec")
                  if p in graphs]
    compare_parts = [p for p in graphs if p not in step_parts]
    ev = {n: [] for n in parts}

    # The step's decode parts are single launches: they go out directly, behind the
    # prefill on the same stream (a graph replay of one launch adds ~20 us of its own);
    # every other part replays its graph.
    eager_in_step = {"decode_get_rows", "decode_mat_vec"}

    def replay(names, record):
        for name in names:
            go = parts[name] if name in eager_in_step else graphs[name].replay
            if record:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                go()
                b.record()
                ev[name].append((a, b))
            else:
                go()

    for _ in range(args.warmup):
        replay(step_parts, False)
    torch.cuda.synchronize()
    log("warm-up done (%d steps)" % args.warmup)

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        replay(step_parts, True)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    log("timed %d steps in %.3f s" % (args.steps, t_total))

    # the other schedules and the widened rows, for comparison (not part of the step)
    replay(compare_parts, False)
    for _ in range(args.steps):
        replay(compare_parts, True)
    torch.cuda.synchronize()
    # the step's decode replayed back to back, as a run of decode tokens would be (in the
    # step it follows the prefill GEMMs on the same GPU)
    b2b = graph_one = None
    if "decode_mat_vec" in graphs:
        graphs["decode_mat_vec"].replay()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(4 * args.steps):
            graphs["decode_mat_vec"].replay()
        b.record()
        torch.cuda.synchronize()
        b2b = a.elapsed_time(b) / (4 * args.steps)
        # and one graph replay at a time, each bracketed by events (the graph's own launch)
        gev = []
        for _ in range(args.steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            graphs["decode_mat_vec"].replay()
            b.record()
            gev.append((a, b))
        torch.cuda.synchronize()
        graph_one = float(np.mean([a.elapsed_time(b) for a, b in gev]))

    # the expert layer's calls, MOE_CALLS of them captured back to back in one graph: the
    # GPU's own time per call (one call per replay would add the ~15-20 us of a graph
    # launch; calls issued one by one from Python would time the host's issue rate, slower
    # than the one-launch decode call itself)
    ms_b2b = {}
    for name in ("expert_layer_prefill", "expert_layer_decode"):
        if name in parts:
            fn = parts[name]
            ms_b2b[name] = graph_ms(torch, lambda: [fn() for _ in range(MOE_CALLS)], args.steps) / MOE_CALLS
    # and at 1, 16, 128 and 512 tokens (the first rows of the prefill's ids), the same way
    moe_by_tokens = {}
    if "expert_layer_prefill" in parts:
        for nt in (1, 16, 128, PREFILL_N):
            ids_nt = moe_ids_p[:nt].contiguous()
            moe_by_tokens[nt] = round(1e3 * graph_ms(
                torch, lambda: [run_moe(ids_nt, B.Q2_0_PREC_F16_MFMA) for _ in range(MOE_CALLS)],
                args.steps) / MOE_CALLS, 2)

    # the decode kernel's own launch time: launches enqueued back to back, an event between
    # each two, so that the GPU finds the next launch queued (no graph launch, no gap)
    launch_us = None
    if "decode_mat_vec" in graphs:
        run_decode_matvecs()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 1)]
        evs[0].record()
        for i in range(2 * args.steps):
            run_decode_matvecs()
            evs[i + 1].record()
        torch.cuda.synchronize()
        launch_us = float(np.mean([evs[i].elapsed_time(evs[i + 1]) for i in range(1, 2 * args.steps)])) * 1e3

    ms = {n: float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in parts if ev[n]}
    ms_stats = {n: {"min": round(float(np.min([a.elapsed_time(b) for a, b in ev[n]])), 4),
                    "median": round(float(np.median([a.elapsed_time(b) for a, b in ev[n]])), 4),
                    "samples": len(ev[n])}
                for n in ("prefill_gemm", "decode_mat_vec", "decode_mat_vec_per_layer") if n in ev and ev[n]}
    if set(step_parts) != {"prefill_get_rows", "prefill_gemm", "decode_get_rows", "decode_mat_vec"}:
        print(json.dumps({"partial_run": True, "ms": ms, "ms_back_to_back": ms_b2b,
                          "expert_layer_us_per_call_by_tokens": moe_by_tokens}), flush=True)
        return

    # ---- algorithmic work
    dec_bytes = sum(mat_bytes(*wl.shapes[n], 1) for (_, n) in order) + mat_bytes(VM, VK, 1)
    f32_flops = sum(2.0 * M * K * PREFILL_N for (_, n) in order[:7] for (M, K) in [wl.shapes[n]])
    pre_flops = sum(2.0 * M * K * PREFILL_N for (_, n) in order for (M, K) in [wl.shapes[n]])
    pre_bytes = sum(mat_bytes(*wl.shapes[n], PREFILL_N) for (_, n) in order)
    matvec_gbs = dec_bytes / (ms["decode_mat_vec"] * 1e-3) / 1e9
    kernel_gbs = dec_bytes / (launch_us * 1e-6) / 1e9
    gemm_tflops = pre_flops / (ms["prefill_gemm"] * 1e-3) / 1e12
    per_layer_gbs = dec_bytes / (ms["decode_mat_vec_per_layer"] * 1e-3) / 1e9
    dec_tok_layer = 1.0 / ((ms["decode_mat_vec_per_layer"] + ms["decode_get_rows"]) * 1e-3)
    dec_tok_stream = 1.0 / ((ms["decode_mat_vec"] + ms["decode_get_rows"]) * 1e-3)
    pre_tok_s = PREFILL_N / ((ms["prefill_gemm"] + ms["prefill_get_rows"]) * 1e-3)
    weight_bytes = sum(stk.host[k].nbytes for k in order)

    traffic = recorded(DECODE_TRAFFIC_PROFILE, "traffic_bytes_per_launch")
    traffic.update(recorded(GEMM_TRAFFIC_PROFILE, "traffic_bytes_per_launch"))
    mfma = recorded(MFMA_PROFILE, "gemm_f16_mfma")
    result = {
        "metric": METRIC,
        "value": round(matvec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_total * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded Q2_0 ternary weights, x ~ N(0,1))",
        "config": {
            "workload": "qwen3_8b_stack_%dx7_plus_vocab151936x4096" % L,
            "layers": L, "decode_N": 1, "prefill_N": PREFILL_N,
            "stack_weight_bytes": weight_bytes, "vocab_bytes": int(emb_host.nbytes),
        },
        "hbm_frac": round(matvec_gbs / HBM_PEAK_GBS, 4),
        "decode_tokens_per_s": round(dec_tok_layer, 1),
        "decode_tokens_per_s_note": "per-layer schedule (q/k/v, o, gate/up, down per layer + head), as a "
                                    "transformer's layer-to-layer dependencies require",
        "decode_tokens_per_s_kernel_stream_bound": round(dec_tok_stream, 1),
        "prefill_tokens_per_s": round(pre_tok_s, 1),
        "prefill_gemm_tflops": round(gemm_tflops, 2),
        "ms": {k: round(v, 4) for k, v in ms.items()},
        "ms_min_median": ms_stats,
        "decode_schedules_GBps": {
            "one batched launch (the step)": round(matvec_gbs, 1),
            "one batched launch, decode tokens back to back (graph replays)":
                round(dec_bytes / (b2b * 1e-3) / 1e9, 1) if b2b else None,
            "one batched launch as a graph replay": round(dec_bytes / (graph_one * 1e-3) / 1e9, 1) if graph_one else None,
            "per_layer_groups (%d launches)" % (len(layer_groups) + 1): round(per_layer_gbs, 1),
            "per_matrix (%d launches)" % (len(order) + 1):
                round(dec_bytes / (ms["decode_mat_vec_per_matrix"] * 1e-3) / 1e9, 1),
        },
        "f32_fallback_gemm_tflops_layer0": round(f32_flops / (ms["prefill_gemm_f32_layer0"] * 1e-3) / 1e12, 2),
        "f32_mfma_gemm_tflops": (round(pre_flops / (ms["prefill_gemm_f32_mfma"] * 1e-3) / 1e12, 1)
                                 if ms.get("prefill_gemm_f32_mfma") else None),
        "f32_mfma_gemm_note": "Q2_0_PREC_F32_MFMA (x as fp16 hi/lo pairs, fp64 block sums, 1e-5 bound under the "
                              "mat-vec's range condition) over the whole prefill (the same 144 group calls)",
        "prefill_schedules_TFLOPs": {
            "per_layer_groups (%d group calls, the step)" % len(prefill_groups): round(gemm_tflops, 1),
            "per_matrix (%d calls)" % len(order):
                round(pre_flops / (ms["prefill_gemm_per_matrix"] * 1e-3) / 1e12, 1),
        },
        "roofline": {
            "kernel": "mat_vec_bcast (N=1, exact limb mode; the step's decode is one launch of 8 items in two "
                      "activation segments: 1.62 GB at K = 4096 in one window, 0.51 GB at K = 12288 in two)",
            "bound": "hbm", "achieved": round(kernel_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kernel_gbs / HBM_PEAK_GBS, 4),
            "traffic": int(traffic["mat_vec_bcast"]) if "mat_vec_bcast" in traffic else None,
            "bytes_per_launch": int(dec_bytes), "avg_launch_us": round(launch_us, 3),
            "note": "achieved = bytes_per_launch / avg_launch_us, the kernel's own launches back to back "
                    "(HIP events between them on their stream); value = the step's decode launch, timed with "
                    "HIP events around it behind the step's prefill",
        },
        "roofline_gemm": {
            "kernel": "gemm_f16_mfma (N=512; %d group calls per prefill, each an fp16 x conversion, one GEMM "
                      "launch and, where K is split, one reduction; achieved over the whole call)" % len(prefill_groups),
            "bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": F16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(gemm_tflops / F16_MFMA_PEAK_TFLOPS, 4),
            "traffic": int(traffic["gemm_f16_prefill"]) if "gemm_f16_prefill" in traffic else None,
            "algorithmic_bytes": int(pre_bytes),
            "mfma_busy_frac_counters": mfma.get("mfma_busy_frac"),
        },
        "next_rows": next_rows(ms, ms_b2b, moe_by_tokens, wl, order, VM, VK, pre_flops, MOE_E, MOE_M, MOE_K,
                               MOE_USED),
        "cpu_baseline": None,
    }
    if not args.no_extra:
        # The step's prefill GEMMs and the comparison schedules leave the GPU at a lower,
        # power-limited clock for a while; the other workloads (several latency-bound)
        # start from an idle GPU, as a separate run of each would.  Clocks are recorded.
        result["gpu_clocks_after_step"] = gpu_clocks()
        torch.cuda.synchronize()
        time.sleep(IDLE_BEFORE_EXTRA_S)
        result["gpu_clocks_before_other_workloads"] = gpu_clocks()
        result["other_workloads"] = other_workloads(torch, dev, B, synth, emb, VM, VK, check, s)
        result["ceilings"] = measured_ceilings(torch, dev, wl, matvec_gbs, gemm_tflops)
    result["gpu_clocks_after_run"] = gpu_clocks()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(stk.host, order, wl, args)

    print(json.dumps(result), flush=True)


IDLE_BEFORE_EXTRA_S = 3.0


def other_workloads(torch, dev, B, synth, emb, VM, VK, check, s):
    """The other configurations, each timed on its own graph (not part of the step):
      * tiny 256 x 512: one mat-vec at N = 1 and get_rows of 4 ids (latency only);
      * Qwen3-1.7B-shaped decode at N = 1 and 8 on a rotation of 56 layer copies (801 MB of
        weights per pass, about three times the 256 MB last-level cache), one batched launch
        per pass and the per-layer schedule;
      * its prefill at N = 512 over 28 layers, per-layer group calls;
      * the 151936 x 4096 vocabulary tensor: get_rows of 512 ids, and the LM head at N = 1
        and 4 rotating over 4 device copies (700 MB, so that the head reads HBM)."""
    out = {}
    reps = 10
    # tiny
    tw = synth.TINY
    M, K = tw.shapes["w"]
    wt = torch.from_numpy(synth.workload_weight(tw, "w")).to(dev)
    xt = torch.from_numpy(synth.activations(tw.seed, 0, 0, 1, K)).to(dev)
    yt = torch.empty((1, M), device=dev)
    idt = torch.from_numpy(synth.row_ids(tw.seed, 0, 0, synth.TINY_IDS, M)).to(dev)
    ot = torch.empty((synth.TINY_IDS, K), device=dev)
    calls = 20   # per graph: one replay per call would time the host's graph submission

    def tiny_mv():
        for _ in range(calls):
            check(B.mul_mat_vec_raw(wt.data_ptr(), M, K, xt.data_ptr(), K, 1, yt.data_ptr(), M, s()), "tiny")

    def tiny_gr():
        for _ in range(calls):
            check(B.get_rows_raw(wt.data_ptr(), M, K, idt.data_ptr(), synth.TINY_IDS, ot.data_ptr(), K, s()), "tiny")
    out["tiny_256x512"] = {
        "mat_vec_N1_us": round(1e3 * graph_ms(torch, tiny_mv, 20) / calls, 2),
        "get_rows_4_us": round(1e3 * graph_ms(torch, tiny_gr, 20) / calls, 2),
        "note": "latency-bound: a few KB of work per call; %d calls per graph, back to back" % calls,
    }
    # Qwen3-1.7B decode, 56-layer rotation
    dw = synth.DECODE_1P7B
    LD = 56
    stk = Stack(torch, dev, dw, LD, synth)
    dec = {}
    for N in (1, 2, 8):
        xs = {K: torch.from_numpy(synth.activations(dw.seed, N, 7 + K // 2048, N, K)).to(dev)
              for K in sorted({K for (_, K) in dw.shapes.values()})}
        ys = {n: torch.empty((N, LD * M), device=dev) for n, (M, K) in dw.shapes.items()}
        ent = [(stk.W[n].data_ptr(), LD * M, K, xs[K].data_ptr(), K, ys[n].data_ptr(), LD * M)
               for n, (M, K) in dw.shapes.items()]
        items = B.make_batch_items(ent)
        groups = []
        for l in range(LD):
            for names in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
                groups.append((B.make_items([(stk.w(l, n).data_ptr(), dw.shapes[n][0],
                                              ys[n][:, l * dw.shapes[n][0]:].data_ptr(), LD * dw.shapes[n][0])
                                             for n in names]), len(names), dw.shapes[names[0]][1]))
        by = LD * sum(mat_bytes(M, K, N) for (M, K) in dw.shapes.values())
        t1 = graph_ms(torch, lambda: check(B.mul_mat_vec_batch_raw(items, len(ent), B.Q2_0_ACT_F32, N, s()),
                                           "1.7b batch"), reps)

        def per_layer():
            st = s()
            for it, n, K in groups:
                check(B.mul_mat_vec_group_raw(it, n, K, xs[K].data_ptr(), K, N, st), "1.7b group")
        t2 = graph_ms(torch, per_layer, reps)
        dec["N%d" % N] = {"one_launch_per_pass_GBps": round(by / (t1 * 1e-3) / 1e9, 1),
                          "per_layer_GBps": round(by / (t2 * 1e-3) / 1e9, 1),
                          "per_layer_tokens_per_s_28_layers": round(N / (t2 * 1e-3 * 28 / LD), 1),
                          "ms_per_pass": [round(t1, 4), round(t2, 4)]}
    dec["note"] = ("56 distinct layer copies (801 MB of weights at N = 1) per pass; tokens/s scaled to the "
                   "model's 28 layers, linear layers only")
    out["qwen3_1p7b_decode"] = dec
    del stk
    # Qwen3-1.7B prefill, 28 layers
    pw = synth.PREFILL_1P7B
    LP = 28
    stk = Stack(torch, dev, pw, LP, synth)
    xP = {K: torch.from_numpy(synth.activations(pw.seed, 0, 7 + K // 2048, PREFILL_N, K)).to(dev)
          for K in sorted({K for (_, K) in pw.shapes.values()})}
    yP = {n: torch.empty((PREFILL_N, M), device=dev) for n, (M, K) in pw.shapes.items()}
    groups = [(B.make_items([(stk.w(l, n).data_ptr(), pw.shapes[n][0], yP[n].data_ptr(), pw.shapes[n][0])
                             for n in names]), len(names), pw.shapes[names[0]][1])
              for l in range(LP) for names in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))]
    wsb = max(B.mul_mat_group_workspace_bytes(it, n, K, PREFILL_N, B.Q2_0_PREC_F16_MFMA) for it, n, K in groups)
    wsp = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)

    def prefill():
        st = s()
        for it, n, K in groups:
            check(B.mul_mat_group_raw(it, n, K, xP[K].data_ptr(), K, PREFILL_N, B.Q2_0_PREC_F16_MFMA,
                                      wsp.data_ptr(), wsb, st), "1.7b prefill")
    tp = graph_ms(torch, prefill, reps)
    flops = LP * sum(2.0 * M * K * PREFILL_N for (M, K) in pw.shapes.values())
    out["qwen3_1p7b_prefill"] = {"TFLOPs": round(flops / (tp * 1e-3) / 1e12, 1),
                                 "frac_of_f16_peak": round(flops / (tp * 1e-3) / 1e12 / F16_MFMA_PEAK_TFLOPS, 4),
                                 "tokens_per_s_28_layers": round(PREFILL_N / (tp * 1e-3), 1), "ms": round(tp, 4)}
    del stk, wsp
    # vocabulary tensor: get_rows and the LM head on 4 rotated copies
    vw = synth.VOCAB_8B
    copies = [emb] + [emb.clone() for _ in range(3)]
    ids = torch.from_numpy(synth.row_ids(vw.seed, 0, 0, synth.VOCAB_IDS, VM)).to(dev)
    og = torch.empty((synth.VOCAB_IDS, VK), device=dev)
    def gr512():
        for _ in range(10):
            check(B.get_rows_raw(emb.data_ptr(), VM, VK, ids.data_ptr(), synth.VOCAB_IDS, og.data_ptr(), VK, s()),
                  "get_rows 512")
    tg = graph_ms(torch, gr512, 10) / 10
    gr_bytes = synth.VOCAB_IDS * (VK // 64 * 18 + 4 * VK + 4)
    vo = {"get_rows_512_GBps": round(gr_bytes / (tg * 1e-3) / 1e9, 1), "get_rows_512_us": round(tg * 1e3, 2)}
    for N in (1, 4):
        xh = torch.from_numpy(synth.activations(vw.seed, N, 0, N, VK)).to(dev)
        yhh = torch.empty((N, VM), device=dev)

        def heads():
            for c in copies:
                check(B.mul_mat_vec_raw(c.data_ptr(), VM, VK, xh.data_ptr(), VK, N, yhh.data_ptr(), VM, s()),
                      "head")
        th = graph_ms(torch, heads, reps) / len(copies)
        vo["lm_head_N%d_GBps" % N] = round(mat_bytes(VM, VK, N) / (th * 1e-3) / 1e9, 1)
        vo["lm_head_N%d_us" % N] = round(th * 1e3, 2)
    vo["lm_head_frac_of_hbm_N1"] = round(vo["lm_head_N1_GBps"] / HBM_PEAK_GBS, 4)
    out["vocab151936x4096"] = vo
    del copies
    torch.cuda.empty_cache()
    return out


def measured_ceilings(torch, dev, wl, matvec_gbs, gemm_tflops):
    """Ceilings measured on this GPU outside the timed region with this repository's own
    measurement kernels (libq2_0_ceilings.so): an HBM read stream over 4 GiB (16-byte loads,
    one 1024-thread workgroup per CU, two loads in flight per thread; plain and non-temporal
    loads), a register-only loop of v_mfma_f32_32x32x16_f16 on pseudo-random operands (no
    memory traffic), and the per-launch cost of an empty kernel in a graph.  For context, a
    dense fp16 GEMM of 8192^3 and the stack's per-layer prefill shapes with fp16 weights on
    hipBLASLt."""
    C = ctypes.CDLL(CEIL_LIB)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    C.q2_0_ceil_read_stream.argtypes = [P, I64, P, I, I, I, I, P]
    C.q2_0_ceil_mfma_f16.argtypes = [I, I, P, P]
    C.q2_0_ceil_empty.argtypes = [P]

    def s():
        return torch.cuda.current_stream().cuda_stream

    def chk(st):
        if st != 0:
            raise RuntimeError("ceiling kernel failed: hipError %d" % st)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3
    out = {}
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.random_(0, 256)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    for nt, key in ((0, "hbm_read_stream_GBps"), (1, "hbm_read_stream_nontemporal_GBps")):
        t = timed(lambda: chk(C.q2_0_ceil_read_stream(buf.data_ptr(), nbytes, sink.data_ptr(), 1024, 256, 2, nt,
                                                      s())), 5)
        out[key] = round(nbytes / t / 1e9, 1)
    del buf
    mo = torch.empty(2048 * 256, dtype=torch.float32, device=dev)
    iters = 2000
    t = timed(lambda: chk(C.q2_0_ceil_mfma_f16(2048, iters, mo.data_ptr(), s())), 3)
    out["mfma_f16_loop_TFLOPs"] = round(2048 * 4 * iters * 4 * 32768 / t / 1e12, 1)
    out["empty_launch_in_graph_us"] = round(1e3 * graph_ms(torch, lambda: [chk(C.q2_0_ceil_empty(s()))
                                                                          for _ in range(100)], 5) / 100, 3)
    a16 = torch.randn((8192, 8192), device=dev, dtype=torch.float16)
    b16 = torch.randn((8192, 8192), device=dev, dtype=torch.float16)
    t = timed(lambda: torch.matmul(a16, b16), 5)
    out["hipblaslt_f16_gemm_8192_TFLOPs"] = round(2 * 8192 ** 3 / t / 1e12, 1)
    del a16, b16
    shapes = [(wl.shapes["q"][0] + 2 * wl.shapes["k"][0], wl.shapes["q"][1]), wl.shapes["o"],
              (2 * wl.shapes["gate"][0], wl.shapes["gate"][1]), wl.shapes["down"]]
    ops = [(torch.randn((PREFILL_N, K), device=dev, dtype=torch.float16),
            torch.randn((K, M), device=dev, dtype=torch.float16) * 0.01) for M, K in shapes]
    t = timed(lambda: [torch.matmul(x16, wt) for x16, wt in ops], 10)
    out["hipblaslt_f16_dense_prefill_layer_TFLOPs"] = round(sum(2.0 * PREFILL_N * M * K for M, K in shapes) / t / 1e12, 1)
    del ops
    out["decode_frac_of_read_stream"] = round(matvec_gbs / out["hbm_read_stream_GBps"], 4)
    out["decode_frac_of_read_stream_nontemporal"] = round(matvec_gbs / out["hbm_read_stream_nontemporal_GBps"], 4)
    out["prefill_frac_of_mfma_loop"] = round(gemm_tflops / out["mfma_f16_loop_TFLOPs"], 4)
    out["note"] = ("read stream, MFMA loop and empty launch: libq2_0_ceilings.so; the hipBLASLt GEMMs are torch's, "
                   "for context")
    return out


def next_rows(ms, ms_b2b, moe_by_tokens, wl, order, VM, VK, pre_flops, ne, mm, mk, nu):
    """Rates of the widened rows, timed beside the step (HIP events around their graphs; the
    expert layer's calls 20 to a graph, ms_b2b, with one call per replay beside)."""
    out = {}

    def rate(name, work, scale, src=None):
        src = ms if src is None else src
        if name in src and src[name] > 0:
            return round(work / (src[name] * 1e-3) / scale, 1)
        return None

    dec16 = sum(M * (K // 64) * 18 + 2 * K + 4 * M for (_, n) in order for (M, K) in [wl.shapes[n]])
    dec16 += VM * (VK // 64) * 18 + 2 * VK + 4 * VM
    out["decode_mat_vec_f16_activations_GBps"] = rate("decode_mat_vec_f16_activations", dec16, 1e9)
    out["prefill_gemm_bf16_activations_TFLOPs"] = rate("prefill_gemm_bf16_activations", pre_flops, 1e12)
    out["quantize_151936x4096_f32_GBps"] = rate("quantize_vocab_f32", VM * VK * 4 + VM * (VK // 64) * 18, 1e9)
    out["repack_g128_151936x4096_GBps"] = rate("repack_g128_vocab", VM * (VK // 128) * 34 + VM * (VK // 64) * 18,
                                              1e9)
    moe_flops = 2.0 * mm * mk * PREFILL_N * nu
    moe_bytes = nu * (mm * (mk // 64) * 18 + 4 * mk + 4 * mm)
    out["expert_layer_prefill_TFLOPs"] = rate("expert_layer_prefill", moe_flops, 1e12, ms_b2b)
    out["expert_layer_decode_GBps"] = rate("expert_layer_decode", moe_bytes, 1e9, ms_b2b)
    out["expert_layer_graph_replay"] = {"prefill_TFLOPs": rate("expert_layer_prefill", moe_flops, 1e12),
                                        "decode_GBps": rate("expert_layer_decode", moe_bytes, 1e9),
                                        "note": "each call as its own graph replay, whose launch (~15-20 us) "
                                                "is timed with it"}
    out["expert_layer"] = ("%d experts of %dx%d, %d per token; prefill %d tokens (fp16 MFMA), decode 1 token "
                           "(fp32-grade mat-vec per pair)" % (ne, mm, mk, nu, PREFILL_N))
    out["ms"] = {k: round(ms[k], 4) for k in ("decode_mat_vec_f16_activations", "prefill_gemm_bf16_activations",
                                              "quantize_vocab_f32", "repack_g128_vocab", "expert_layer_prefill",
                                              "expert_layer_decode") if k in ms}
    out["ms_expert_layer_back_to_back"] = {k: round(v, 4) for k, v in ms_b2b.items()}
    out["expert_layer_back_to_back_note"] = "20 calls captured back to back in one graph, ms per call"
    out["expert_layer_us_per_call_by_tokens"] = {str(k): v for k, v in moe_by_tokens.items()}
    return out


def gpu_clocks() -> dict:
    """The GPU's current and available sclk / mclk as rocm-smi reports them (read-only
    query; None where the tool or a field is missing)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        d = json.loads(r.stdout)
    except Exception:
        return {"sclk": None, "mclk": None}
    card = next(iter(d.values()), {}) if isinstance(d, dict) else {}
    pick = lambda key: next((v for k, v in card.items() if key in k.lower()), None)
    return {"sclk": pick("sclk"), "mclk": pick("mclk")}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(host_w, order, wl, args):
    """The fp64 oracle, as it stands, on the host cores: the decode mat-vec over the whole
    stack at N = 1 and the prefill product on every S-th row of every matrix at N = 512; and
    on one thread, the tiny case, one Qwen3-1.7B decode layer at N = 1 and that layer's
    prefill at N = 512 on every 64th row."""
    import oracle
    from ternary_bit_quantized_amd import synth
    oracle.build()
    threads = oracle.num_threads()
    xs1 = {K: synth.activations(wl.seed, 0, synth.stack_x_matrix_index(K), 1, K) for K in (4096, 12288)}
    xsP = {K: synth.activations(wl.seed, 1, synth.stack_x_matrix_index(K), PREFILL_N, K) for K in (4096, 12288)}
    t = time.perf_counter()
    nbytes = 0
    for _ in range(args.cpu_decode_repeats):
        for key in order:
            M, K = wl.shapes[key[1]]
            oracle.mul_mat(host_w[key], M, K, xs1[K])
            nbytes += mat_bytes(M, K, 1)
    t_dec = (time.perf_counter() - t) / args.cpu_decode_repeats
    nbytes //= args.cpu_decode_repeats
    log("cpu oracle decode: %.2f s" % t_dec)
    S = args.cpu_prefill_row_stride
    t = time.perf_counter()
    flops = 0.0
    for key in order:
        M, K = wl.shapes[key[1]]
        rows = np.arange(0, M, S)
        oracle.mul_mat(host_w[key], M, K, xsP[K], rows=rows)
        flops += 2.0 * rows.size * K * PREFILL_N
    t_pre = time.perf_counter() - t
    log("cpu oracle prefill sample: %.2f s" % t_pre)
    # one thread
    one = {}
    oracle.set_num_threads(1)
    try:
        tw = synth.TINY
        M, K = tw.shapes["w"]
        w = synth.workload_weight(tw, "w")
        x = synth.activations(tw.seed, 0, 0, 1, K)
        t = time.perf_counter()
        for _ in range(200):
            oracle.mul_mat(w, M, K, x)
        one["tiny_mat_vec_us"] = round((time.perf_counter() - t) / 200 * 1e6, 1)
        dw = synth.DECODE_1P7B
        mats = {n: synth.workload_weight(dw, n, 0) for n in synth.MATS}
        xd = {K: synth.activations(dw.seed, 0, 7, 1, K) for K in (2048, 6144)}
        t = time.perf_counter()
        by = 0
        for n in synth.MATS:
            M, K = dw.shapes[n]
            oracle.mul_mat(mats[n], M, K, xd[K])
            by += mat_bytes(M, K, 1)
        td = time.perf_counter() - t
        one["qwen3_1p7b_decode_layer_GBps"] = round(by / td / 1e9, 4)
        xp = {K: synth.activations(dw.seed, 1, 7, PREFILL_N, K) for K in (2048, 6144)}
        t = time.perf_counter()
        fl = 0.0
        for n in synth.MATS:
            M, K = dw.shapes[n]
            rows = np.arange(0, M, 64)
            oracle.mul_mat(mats[n], M, K, xp[K], rows=rows)
            fl += 2.0 * rows.size * K * PREFILL_N
        one["qwen3_1p7b_prefill_layer_GFLOPs_rows_1_in_64"] = round(fl / (time.perf_counter() - t) / 1e9, 3)
    finally:
        oracle.set_num_threads(threads)
    log("cpu oracle single-thread figures done")
    return {
        "value": round(nbytes / t_dec / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": "decode mat-vec N=1 over all %d stack matrices (%d B), mean of %d passes; prefill "
                  "N=512 on every %dth row of each matrix" % (len(order), nbytes, args.cpu_decode_repeats, S),
        "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
        "decode_s": round(t_dec, 3), "prefill_sample_s": round(t_pre, 3),
        "prefill_tflops": round(flops / t_pre / 1e12, 6),
        "decode_tokens_per_s": round(1.0 / t_dec, 4),
        "one_thread": one,
    }


if __name__ == "__main__":
    main()
