"""Benchmark of the Q2_0 hot path on one MI355X.

Workload: a Qwen3-8B-shaped ternary model's linear work -- the 36-layer stack of
q/o 4096x4096, k/v 1024x4096, gate/up 12288x4096 and down 4096x12288 Q2_0 matrices
(1.95 GB) plus a 151936x4096 Q2_0 vocabulary tensor used both as the embedding
(get_rows) and as the LM head -- with seeded synthetic weights and activations.

One step is one pass of the whole hot path:
  prefill: get_rows of 512 token ids, then the 252 stack matrices at N = 512 on the
           fp16-MFMA GEMM, per layer as the model runs them: q/k/v as one group call
           (they share the input), o, gate/up as one group call, down;
  decode : get_rows of 1 token id, then the 252 stack matrices and the LM head at
           N = 1 on the mat-vec (one token, weights streamed from HBM).  The stack's
           matrices use one activation per distinct K, so they are launched grouped by
           activation (64 matrices a launch): the K = 4096 matrices, the K = 12288
           matrices, then the head, alternating between two streams (the launches are
           independent, so one launch's drain overlaps the next one's ramp-up).
Each part is captured once in a HIP graph and replayed, so the timed region holds
GPU work only.  Inputs are resident in HBM before timing starts.

The same decode is also timed, outside the step, under two other launch schedules:
per layer as a transformer with layer-to-layer dependencies would run it (grouped
q/k/v, o, grouped gate/up, down: 4 launches per layer + head) and one launch per
matrix.  Every launch here costs a few microseconds of ramp-up and drain, which
bounds those schedules whatever the kernel does.

Printed: one JSON line.  `value` is the decode mat-vec stream rate in GB/s
(algorithmic bytes: Q2_0 weights + f32 activations + f32 outputs, over the time of
the decode mat-vec launches).  Extra fields give decode and prefill tokens/s, the
prefill GEMM TFLOP/s, the roofline fractions, the other decode schedules, the fp32
fallback GEMM's rate on one layer, and the CPU oracle's rate on a bounded sample of
the same work.

Profiling: --eager launches the selected --parts directly (no graphs), and
--copy-calibration-mib runs one elementwise copy-like kernel (torch.neg) of known
size first, whose counter readings scale the kernels' FETCH_SIZE / WRITE_SIZE to
bytes.
"""

from __future__ import annotations

import argparse
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


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "mat_vec_bcast_gemm_f16_hbm_traffic.md")


def kernel_sources_sha256() -> str:
    """sha256 over the code of the HIP sources of libq2_0.so (sorted by name; comments and
    blank lines removed, so that a comment edit keeps it), to tell whether the recorded
    counter readings still describe the kernels being timed."""
    import hashlib
    import re
    h = hashlib.sha256()
    src = os.path.join(ROOT, "ternary_bit_quantized_amd", "csrc")
    for name in sorted(os.listdir(src)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(src, name), encoding="utf-8") as f:
                text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
            code = "\n".join(ln.rstrip() for ln in (re.sub(r"//.*", "", l) for l in text.splitlines()) if ln.strip())
            h.update(name.encode() + b"\0" + code.encode())
    return h.hexdigest()


def recorded_traffic() -> dict:
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE passes
    (lines `traffic_bytes_per_launch <kernel>: <bytes>`), or {} when the kernel sources
    changed after those passes were taken (line `sources_sha256: <hex>`)."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return {}
    out, sha = {}, None
    for ln in lines:
        ln = ln.strip().strip("`")
        if ln.startswith("sources_sha256:"):
            sha = ln.split(":", 1)[1].strip()
        elif ln.startswith("traffic_bytes_per_launch "):
            key, val = ln[len("traffic_bytes_per_launch "):].split(":", 1)
            out[key.strip()] = int(val)
    return out if sha == kernel_sources_sha256() else {}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=36, help="stack layers (36 = the full model)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-prefill-row-stride", type=int, default=16)
    p.add_argument("--cpu-decode-repeats", type=int, default=8)
    p.add_argument("--eager", action="store_true", help="launch parts directly, without HIP graphs")
    p.add_argument("--parts", default="", help="comma-separated subset of parts to run (profiling)")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="one device-to-device copy of this size before the parts (counter scaling)")
    return p.parse_args()


def mat_bytes(M, K, N):
    return M * (K // 64) * 18 + 4 * K * N + 4 * M * N


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
    layers = list(range(args.layers))
    t0 = time.time()
    host_w = synth.stack_weights(wl, layers, threads=min(16, os.cpu_count() or 8))
    emb_host = synth.workload_weight(vwl, "emb")
    log("generated %d matrices + vocab tensor in %.1f s" % (len(host_w), time.time() - t0))

    W = {k: torch.from_numpy(v).to(dev) for k, v in host_w.items()}
    emb = torch.from_numpy(emb_host).to(dev)
    VM, VK = vwl.shapes["emb"]
    Ks = sorted({K for (_, K) in wl.shapes.values()})
    Ms = sorted({M for (M, _) in wl.shapes.values()} | {VM})
    x1 = {K: torch.from_numpy(synth.activations(wl.seed, 0, synth.stack_x_matrix_index(K), 1, K)).to(dev)
          for K in Ks}
    xP = {K: torch.from_numpy(synth.activations(wl.seed, 1, synth.stack_x_matrix_index(K), PREFILL_N, K)).to(dev)
          for K in Ks}
    y1 = {M: torch.empty((1, M), dtype=torch.float32, device=dev) for M in Ms}
    ids_p = torch.from_numpy(synth.row_ids(vwl.seed, 0, 0, PREFILL_N, VM)).to(dev)
    ids_d = torch.from_numpy(synth.row_ids(vwl.seed, 1, 0, 1, VM)).to(dev)
    emb_out_p = torch.empty((PREFILL_N, VK), dtype=torch.float32, device=dev)
    emb_out_d = torch.empty((1, VK), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log("inputs resident on the GPU")

    order = [(l, n) for l in layers for n in synth.MATS]

    def check(st, what):
        if st != 0:
            raise RuntimeError("%s failed: %s" % (what, B.lib().q2_0_status_string(st).decode()))

    def s():
        return torch.cuda.current_stream().cuda_stream

    def run_get_rows(ids, out):
        check(B.get_rows_raw(emb.data_ptr(), VM, VK, ids.data_ptr(), ids.numel(), out.data_ptr(), VK, s()),
              "get_rows")

    # one output buffer per matrix so grouped launches never share a y
    yd = {key: torch.empty((1, wl.shapes[key[1]][0]), dtype=torch.float32, device=dev) for key in order}

    def head(st):
        check(B.mul_mat_vec_raw(emb.data_ptr(), VM, VK, x1[VK].data_ptr(), VK, 1, y1[VM].data_ptr(), VM, st),
              "lm_head")

    def run_decode_per_matrix():
        st = s()
        for key in order:
            M, K = wl.shapes[key[1]]
            check(B.mul_mat_vec_raw(W[key].data_ptr(), M, K, x1[K].data_ptr(), K, 1,
                                    yd[key].data_ptr(), M, st), "mat_vec")
        head(st)

    def group_items(keys):
        return B.make_items([(W[k].data_ptr(), wl.shapes[k[1]][0], yd[k].data_ptr(), wl.shapes[k[1]][0])
                             for k in keys])

    layer_groups = []
    for l in layers:
        for names in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
            keys = [(l, n) for n in names]
            layer_groups.append((group_items(keys), len(keys), wl.shapes[names[0]][1]))
    by_k = {}
    for key in order:
        by_k.setdefault(wl.shapes[key[1]][1], []).append(key)

    def run_groups(groups):
        st = s()
        for items, n, K in groups:
            check(B.mul_mat_vec_group_raw(items, n, K, x1[K].data_ptr(), K, 1, st), "mat_vec_group")
        head(st)

    # The by-activation decode: one launch per 64 matrices of one activation (the
    # library's group limit), then the head.  The launches are independent products, so
    # they alternate between the capture stream and a second stream (default priority),
    # joined at the end: one launch's tail overlaps the next one's ramp.
    side2 = torch.cuda.Stream()
    act_chunks = []
    for K, keys in sorted(by_k.items()):
        for c in range(0, len(keys), 64):
            act_chunks.append((group_items(keys[c:c + 64]), len(keys[c:c + 64]), K))

    def run_two_streams(launches):
        cur = torch.cuda.current_stream()
        side2.wait_stream(cur)
        for i, fn in enumerate(launches):
            fn((cur if i % 2 == 0 else side2).cuda_stream)
        cur.wait_stream(side2)

    def run_decode_matvecs():
        run_two_streams([(lambda st, it=it, n=n, K=K: check(
            B.mul_mat_vec_group_raw(it, n, K, x1[K].data_ptr(), K, 1, st), "mat_vec_group"))
            for it, n, K in act_chunks] + [head])

    # prefill: one output buffer per matrix name (grouped items never share a y); the
    # layer's matrices that share x run as one group: q/k/v, o, gate/up, down
    yPn = {n: torch.empty((PREFILL_N, wl.shapes[n][0]), dtype=torch.float32, device=dev) for n in synth.MATS}
    prefill_names = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))

    def prefill_items(l, names):
        return B.make_items([(W[(l, n)].data_ptr(), wl.shapes[n][0], yPn[n].data_ptr(), wl.shapes[n][0])
                             for n in names])

    prefill_groups = [(prefill_items(l, names), len(names), wl.shapes[names[0]][1])
                      for l in layers for names in prefill_names]
    ws_bytes = max(max(B.mul_mat_group_workspace_bytes(items, n, K, PREFILL_N, B.Q2_0_PREC_F16_MFMA)
                       for (items, n, K) in prefill_groups),
                   max(B.mul_mat_workspace_bytes(M, K, PREFILL_N, B.Q2_0_PREC_F16_MFMA)
                       for (M, K) in wl.shapes.values()))
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def run_prefill_gemms(precision=B.Q2_0_PREC_F16_MFMA, groups=None):
        st = s()
        for items, n, K in (groups or prefill_groups):
            check(B.mul_mat_group_raw(items, n, K, xP[K].data_ptr(), K, PREFILL_N, precision,
                                      ws.data_ptr(), ws_bytes, st), "mul_mat_group")

    def run_prefill_per_matrix():
        st = s()
        for key in order:
            M, K = wl.shapes[key[1]]
            check(B.mul_mat_raw(W[key].data_ptr(), M, K, xP[K].data_ptr(), K, PREFILL_N,
                                yPn[key[1]].data_ptr(), M, B.Q2_0_PREC_F16_MFMA, ws.data_ptr(), ws_bytes, st),
                  "mul_mat")

    # ---- the widened rows, measured beside the step (not part of it): 16-bit activations,
    # the quantizer and the legacy group-128 reader, an expert layer
    x1h = {K: v.to(torch.float16) for K, v in x1.items()}
    xPb = {K: v.to(torch.bfloat16) for K, v in xP.items()}

    def run_decode_f16_activations():
        run_two_streams([(lambda st, it=it, n=n, K=K: check(
            B.mul_mat_vec_group_act_raw(it, n, K, x1h[K].data_ptr(), B.Q2_0_ACT_F16, K, 1, st), "mat_vec_group_act"))
            for it, n, K in act_chunks] + [lambda st: check(
                B.mul_mat_vec_act_raw(emb.data_ptr(), VM, VK, x1h[VK].data_ptr(), B.Q2_0_ACT_F16, VK, 1,
                                      y1[VM].data_ptr(), VM, st), "lm_head_act")])

    def run_prefill_bf16_activations():
        st = s()
        for items, n, K in prefill_groups:
            check(B.mul_mat_group_act_raw(items, n, K, xPb[K].data_ptr(), B.Q2_0_ACT_BF16, K, PREFILL_N,
                                          B.Q2_0_PREC_F16_MFMA, ws.data_ptr(), ws_bytes, st), "mul_mat_group_act")

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
    # them per token; prefill 512 tokens on the fp16 GEMM, decode one token on the fp32 path
    MOE_E, MOE_M, MOE_K, MOE_USED = 128, 768, 2048, 8
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

    # ---- capture the parts as graphs
    parts = {
        "prefill_get_rows": lambda: run_get_rows(ids_p, emb_out_p),
        "prefill_gemm": run_prefill_gemms,
        "decode_get_rows": lambda: run_get_rows(ids_d, emb_out_d),
        "decode_mat_vec": run_decode_matvecs,
        "decode_mat_vec_per_layer": lambda: run_groups(layer_groups),
        "decode_mat_vec_per_matrix": run_decode_per_matrix,
        "prefill_gemm_per_matrix": run_prefill_per_matrix,
        "prefill_gemm_f32_layer0": lambda: run_prefill_gemms(B.Q2_0_PREC_F32, groups=prefill_groups[:4]),
        "decode_mat_vec_f16_activations": run_decode_f16_activations,
        "prefill_gemm_bf16_activations": run_prefill_bf16_activations,
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
    graphs = {}
    if args.eager:
        for name, fn in parts.items():
            fn()
        torch.cuda.synchronize()
        log("eager parts done: %s" % ",".join(parts))
        return
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
    compare_parts = [p for p in ("decode_mat_vec_per_layer", "decode_mat_vec_per_matrix",
                                 "prefill_gemm_per_matrix", "prefill_gemm_f32_layer0",
                                 "decode_mat_vec_f16_activations", "prefill_gemm_bf16_activations",
                                 "quantize_vocab_f32", "repack_g128_vocab", "expert_layer_prefill",
                                 "expert_layer_decode") if p in graphs]
    ev = {n: [] for n in parts}

    def replay(names, record):
        for name in names:
            g = graphs[name]
            if record:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                ev[name].append((a, b))
            else:
                g.replay()

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

    # the other decode schedules and the fp32 fallback, for comparison (not part of the step)
    replay(compare_parts, False)
    for _ in range(args.steps):
        replay(compare_parts, True)
    torch.cuda.synchronize()
    # the step's decode replayed back to back, as a run of decode tokens would be (in the
    # step it follows 11 ms of prefill GEMM on the same GPU)
    b2b = None
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

    ms = {n: float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in parts if ev[n]}
    if set(step_parts) != {"prefill_get_rows", "prefill_gemm", "decode_get_rows", "decode_mat_vec"}:
        print(json.dumps({"partial_run": True, "ms": ms}), flush=True)
        return

    # ---- algorithmic work
    dec_bytes = sum(mat_bytes(*wl.shapes[n], 1) for (_, n) in order) + mat_bytes(VM, VK, 1)
    n_dec_launches = len(act_chunks) + 1
    f32_flops = sum(2.0 * M * K * PREFILL_N for (_, n) in order[:7] for (M, K) in [wl.shapes[n]])
    pre_flops = sum(2.0 * M * K * PREFILL_N for (_, n) in order for (M, K) in [wl.shapes[n]])
    pre_bytes = sum(mat_bytes(*wl.shapes[n], PREFILL_N) for (_, n) in order)
    matvec_gbs = dec_bytes / (ms["decode_mat_vec"] * 1e-3) / 1e9
    gemm_tflops = pre_flops / (ms["prefill_gemm"] * 1e-3) / 1e12
    dec_tok_s = 1.0 / ((ms["decode_mat_vec"] + ms["decode_get_rows"]) * 1e-3)
    pre_tok_s = PREFILL_N / ((ms["prefill_gemm"] + ms["prefill_get_rows"]) * 1e-3)
    weight_bytes = sum(host_w[k].nbytes for k in order)

    traffic = recorded_traffic()
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
            "workload": "qwen3_8b_stack_%dx7_plus_vocab151936x4096" % args.layers,
            "layers": args.layers, "decode_N": 1, "prefill_N": PREFILL_N,
            "stack_weight_bytes": weight_bytes, "vocab_bytes": int(emb_host.nbytes),
        },
        "hbm_frac": round(matvec_gbs / HBM_PEAK_GBS, 4),
        "decode_tokens_per_s": round(dec_tok_s, 1),
        "prefill_tokens_per_s": round(pre_tok_s, 1),
        "prefill_gemm_tflops": round(gemm_tflops, 2),
        "ms": {k: round(v, 4) for k, v in ms.items()},
        "decode_schedules_GBps": {
            "by_activation (%d launches on two streams, the step)" % n_dec_launches: round(matvec_gbs, 1),
            "by_activation, decode tokens back to back": round(dec_bytes / (b2b * 1e-3) / 1e9, 1) if b2b else None,
            "per_layer_groups (%d launches)" % (len(layer_groups) + 1):
                round(dec_bytes / (ms["decode_mat_vec_per_layer"] * 1e-3) / 1e9, 1),
            "per_matrix (%d launches)" % (len(order) + 1):
                round(dec_bytes / (ms["decode_mat_vec_per_matrix"] * 1e-3) / 1e9, 1),
        },
        "decode_tokens_per_s_per_layer_schedule": round(
            1.0 / ((ms["decode_mat_vec_per_layer"] + ms["decode_get_rows"]) * 1e-3), 1),
        "f32_fallback_gemm_tflops_layer0": round(f32_flops / (ms["prefill_gemm_f32_layer0"] * 1e-3) / 1e12, 2),
        "prefill_schedules_TFLOPs": {
            "per_layer_groups (%d group calls, the step)" % len(prefill_groups): round(gemm_tflops, 1),
            "per_matrix (%d calls)" % len(order):
                round(pre_flops / (ms["prefill_gemm_per_matrix"] * 1e-3) / 1e12, 1),
        },
        "roofline": {
            "kernel": "mat_vec_bcast (N=1; %d grouped launches per decode token on two streams: exact mode "
                      "where K <= 8192, hi/lo mode at K = 12288; avg_launch_us = the decode graph's time / "
                      "launches)" % n_dec_launches,
            "bound": "hbm", "achieved": round(matvec_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(matvec_gbs / HBM_PEAK_GBS, 4), "traffic": traffic.get("mat_vec_bcast"),
            "bytes_per_launch_avg": int(dec_bytes / n_dec_launches),
            "avg_launch_us": round(ms["decode_mat_vec"] * 1e3 / n_dec_launches, 3),
        },
        "roofline_gemm": {
            "kernel": "gemm_f16_mfma (N=512; %d group calls per prefill, each an fp16 x conversion, "
                      "one GEMM launch and, where K is split, one reduction)" % len(prefill_groups),
            "bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": F16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(gemm_tflops / F16_MFMA_PEAK_TFLOPS, 4),
            "traffic": traffic.get("gemm_f16_mfma"), "algorithmic_bytes": int(pre_bytes),
        },
        "next_rows": next_rows(ms, wl, order, VM, VK, pre_flops, MOE_E, MOE_M, MOE_K, MOE_USED),
        "cpu_baseline": None,
    }

    result["ceilings"] = measured_ceilings(dev, wl, matvec_gbs, gemm_tflops)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(host_w, order, wl, args)

    print(json.dumps(result), flush=True)


def measured_ceilings(dev, wl, matvec_gbs, gemm_tflops):
    """Context for the roofline fractions, measured on this GPU outside the timed region with
    torch's own kernels (not this library): a 2 GiB device copy (HBM read + write rate), a
    dense fp16 GEMM of 8192^3 (hipBLASLt), and the stack's per-layer prefill shapes as dense
    fp16 GEMMs (the weights as fp16, 7.1x the bytes of Q2_0) at N = 512.  Random operands."""
    import torch

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
    n = (2 << 30) // 4
    src = torch.randn(n, device=dev)
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src), 5)
    out["hbm_copy_GBps"] = round(2 * 4 * n / t / 1e9, 1)
    del src, dst
    a16 = torch.randn((8192, 8192), device=dev, dtype=torch.float16)
    b16 = torch.randn((8192, 8192), device=dev, dtype=torch.float16)
    t = timed(lambda: torch.matmul(a16, b16), 5)
    out["f16_gemm_8192_TFLOPs"] = round(2 * 8192 ** 3 / t / 1e12, 1)
    del a16, b16
    shapes = [(wl.shapes["q"][0] + 2 * wl.shapes["k"][0], wl.shapes["q"][1]), wl.shapes["o"],
              (2 * wl.shapes["gate"][0], wl.shapes["gate"][1]), wl.shapes["down"]]
    ops = []
    for M, K in shapes:
        x16 = torch.randn((PREFILL_N, K), device=dev, dtype=torch.float16)
        wt = torch.randn((K, M), device=dev, dtype=torch.float16) * 0.01
        ops.append((x16, wt))
    t = timed(lambda: [torch.matmul(x16, wt) for x16, wt in ops], 10)
    flops = sum(2.0 * PREFILL_N * M * K for M, K in shapes)
    out["f16_dense_prefill_layer_TFLOPs"] = round(flops / t / 1e12, 1)
    del ops
    out["decode_frac_of_copy_rate"] = round(matvec_gbs / out["hbm_copy_GBps"], 4)
    out["prefill_frac_of_f16_gemm_8192"] = round(gemm_tflops / out["f16_gemm_8192_TFLOPs"], 4)
    out["note"] = ("torch's own kernels on this GPU, outside the timed region: an elementwise copy, hipBLASLt "
                   "fp16 GEMMs (8192^3, and the stack's q/k/v, o, gate/up, down shapes at N = 512 with fp16 "
                   "weights)")
    return out


def next_rows(ms, wl, order, VM, VK, pre_flops, ne, mm, mk, nu):
    """Rates of the widened rows, timed beside the step (HIP events around their graphs)."""
    out = {}

    def rate(name, work, scale):
        if name in ms and ms[name] > 0:
            return round(work / (ms[name] * 1e-3) / scale, 1)
        return None

    dec16 = sum(M * (K // 64) * 18 + 2 * K + 4 * M for (_, n) in order for (M, K) in [wl.shapes[n]])
    dec16 += VM * (VK // 64) * 18 + 2 * VK + 4 * VM
    out["decode_mat_vec_f16_activations_GBps"] = rate("decode_mat_vec_f16_activations", dec16, 1e9)
    out["prefill_gemm_bf16_activations_TFLOPs"] = rate("prefill_gemm_bf16_activations", pre_flops, 1e12)
    out["quantize_151936x4096_f32_GBps"] = rate("quantize_vocab_f32", VM * VK * 4 + VM * (VK // 64) * 18, 1e9)
    out["repack_g128_151936x4096_GBps"] = rate("repack_g128_vocab", VM * (VK // 128) * 34 + VM * (VK // 64) * 18,
                                              1e9)
    out["expert_layer_prefill_TFLOPs"] = rate("expert_layer_prefill", 2.0 * mm * mk * PREFILL_N * nu, 1e12)
    out["expert_layer_decode_GBps"] = rate("expert_layer_decode", nu * (mm * (mk // 64) * 18 + 4 * mk + 4 * mm), 1e9)
    out["expert_layer"] = "%d experts of %dx%d, %d per token; prefill %d tokens (fp16 MFMA), decode 1 token (fp32)" % (
        ne, mm, mk, nu, PREFILL_N)
    out["ms"] = {k: round(ms[k], 4) for k in ("decode_mat_vec_f16_activations", "prefill_gemm_bf16_activations",
                                              "quantize_vocab_f32", "repack_g128_vocab", "expert_layer_prefill",
                                              "expert_layer_decode") if k in ms}
    return out


def cpu_baseline(host_w, order, wl, args):
    """The fp64 oracle, as it stands, on the host cores: the decode mat-vec over the whole
    stack at N = 1 and the prefill product on every S-th row of every matrix at N = 512."""
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
    return {
        "value": round(nbytes / t_dec / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": "decode mat-vec N=1 over all %d stack matrices (%d B), mean of %d passes; prefill "
                  "N=512 on every %dth row of each matrix" % (len(order), nbytes, args.cpu_decode_repeats, S),
        "decode_s": round(t_dec, 3), "prefill_sample_s": round(t_pre, 3),
        "prefill_tflops": round(flops / t_pre / 1e12, 6),
        "decode_tokens_per_s": round(1.0 / t_dec, 4),
    }


if __name__ == "__main__":
    main()
