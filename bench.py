#!/usr/bin/env python3
"""Benchmark of the W4A16 grouped-quantized MoE layer on one MI355X.

Headline workload (one "step" = one decode token through one Ling-shape MoE
layer: route + gate_up/SiLU + down + weighted combine + shared expert, M = 1):
  hidden 2560, 512 routed experts, top-8, moe_intermediate 768, INT4 g32
  routed experts with bf16 scales, bf16 shared expert, fp32 router.
Steps rotate over C resident copies of the layer (distinct device memory,
distinct seeded routers), so a step never finds its weights in the 256 MB
last-level cache; the step chain is captured in HIP graphs and replayed.
Throughput is algorithmic bytes per step / time (GB/s) and microseconds per
token.

Timing: W warm-up steps, then the K timed steps (exactly K) are replayed
between HIP events on the launch stream, behind one untimed replay that keeps
the GPU busy while the host enqueues them (so the region holds GPU work
only); this is done three times and the median is reported, with each run's
time beside it.

The same run also measures, each with its own roofline (key "extra"): the
speculative-verify steps (M = 2 and 4 tokens), one token through 40 stacked
layers with RMSNorm between them, one 4096-token prefill chunk, the LM head
for one token as FP8 and as BF16 (157,184 x 2,560), the decode step with
the routed experts in MXFP4 and in block FP8, and a speculative-decoding
round (3 draft steps and a 4-position verify on the 40-layer stack, with the
verify:decode ratio); the HBM
read rate a plain streaming kernel reaches on this part (the achievable
ceiling); and the CPU oracle on this host's cores and on one core.

--workload selects a different headline (then no extras are measured).
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0

# Algorithmic bytes (Ling shape): every weight byte a step must read once,
# plus activations in and out.
EXPERT_GU_BYTES = 2 * 768 * 2560 // 2 + 2 * 768 * (2560 // 32) * 2     # 2,211,840
EXPERT_DN_BYTES = 2560 * 768 // 2 + 2560 * (768 // 32) * 2             # 1,105,920
EXPERT_BYTES = EXPERT_GU_BYTES + EXPERT_DN_BYTES                        # 3,317,760
SHARED_GU_BYTES = 2 * 768 * 2560 * 2                                    # 7,864,320
SHARED_DN_BYTES = 2560 * 768 * 2                                        # 3,932,160
ROUTER_BYTES = 512 * 2560 * 4                                           # 5,242,880
TOKEN_IO_BYTES = 2 * 2560 * 2                                           # x in, out back
STACK_LAYERS = 40

WORKLOAD_NAMES = {"decode": "ling_moe_layer_decode_m1", "verify2": "ling_moe_layer_verify_m2",
                  "verify4": "ling_moe_layer_verify_m4", "stack": "ling_moe_stack40_decode_m1",
                  "prefill": "ling_moe_layer_prefill_m4096",
                  "lmhead_fp8": "ling_lm_head_fp8_m1", "lmhead_bf16": "ling_lm_head_bf16_m1",
                  "decode_mxfp4": "ling_moe_layer_mxfp4_decode_m1", "decode_fp8block": "ling_moe_layer_fp8block_decode_m1",
                  "mtp_round": "ling_moe_stack40_mtp_round_3drafts"}
TOKENS = {"decode": 1, "verify2": 2, "verify4": 4, "stack": 1, "prefill": 4096, "lmhead_fp8": 1, "lmhead_bf16": 1,
          "decode_mxfp4": 1, "decode_fp8block": 1, "mtp_round": 4}
# (timed steps, warm-up steps) of the extra workloads measured beside the headline
EXTRA_STEPS = {"verify2": (256, 32), "verify4": (256, 32), "stack": (16, 4), "prefill": (8, 2),
               "lmhead_fp8": (256, 16), "lmhead_bf16": (128, 8), "decode_mxfp4": (512, 64),
               "decode_fp8block": (512, 64), "mtp_round": (16, 2)}
# accept length per round the pages report for 3 draft steps (bpdata.com
# article, "Optimalizáció 3")
MTP_ACCEPT = 3.90
# bytes of one routed expert in the other formats: codes + scales of gate_up and down
EXPERT_BYTES_FMT = {"decode_mxfp4": 2 * 768 * (2560 // 2 + 2560 // 32) + 2560 * (768 // 2 + 768 // 32),
                    "decode_fp8block": 2 * 768 * 2560 + 12 * 20 * 4 + 2560 * 768 + 20 * 6 * 4}
FMT_COPIES = 8
LM_HIDDEN = 2560


def step_bytes(n_unique_experts: int, M: int) -> int:
    return n_unique_experts * EXPERT_BYTES + SHARED_GU_BYTES + SHARED_DN_BYTES + ROUTER_BYTES + M * TOKEN_IO_BYTES


def prefill_flops(M: int, k: int = 8) -> float:
    """Expert flops of one chunk: routed pairs and the shared expert, gate_up
    (2 x 768 x 2560) and down (2560 x 768) multiply-adds each."""
    per = 2 * 768 * 2560 + 2560 * 768
    return 2.0 * M * k * per + 2.0 * M * per


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2048)
    p.add_argument("--warmup", type=int, default=256)
    p.add_argument("--workload", default="decode", choices=list(WORKLOAD_NAMES))
    p.add_argument("--copies", type=int, default=32,
                   help="resident layer copies the decode/verify steps rotate over (prefill uses one)")
    p.add_argument("--chunk", type=int, default=256, help="decode/verify steps captured per graph")
    p.add_argument("--runs", type=int, default=3, help="timed runs of K steps; the median is reported")
    p.add_argument("--path", default="layer", choices=["layer", "calls"],
                   help="layer: one moe_layer_w4a16 call per layer step (one launch at M = 1); "
                        "calls: moe_route then moe_forward_w4a16")
    p.add_argument("--no-extras", action="store_true", help="measure the headline workload only")
    p.add_argument("--cpu-baseline-seconds", type=float, default=12.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--stage-steps", type=int, default=256, help="launches per graph when timing one entry point")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="after timing, run a plain device copy of this many MiB (reference for HBM byte counters)")
    return p.parse_args(argv)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Ctx:
    """Device state shared by the workloads of one run."""

    def __init__(self, args, n_copies):
        import torch

        from w4a16_grouped_quantized_amd import binding as B
        from w4a16_grouped_quantized_amd import synth
        self.torch, self.B, self.synth, self.args = torch, B, synth, args
        self.shape = synth.LING
        self.cfg = B.config(self.shape)
        t0 = time.time()
        self.layer = synth.make_layer(self.shape, 1, threads=16)
        base = B.MoeLayer(self.layer)
        log(f"layer generated and packed in {time.time() - t0:.1f}s; build: {B.build_info()}")
        # copies: distinct device memory; distinct seeded routers (layer seeds 1000 + c)
        self.copies = []
        for c in range(n_copies):
            packed = base.packed if c == 0 else base.packed.clone()
            router = torch.from_numpy(synth.make_router(self.shape, 1000 + c)).cuda()
            self.copies.append((packed, router))
        torch.cuda.synchronize()
        log(f"{n_copies} resident copies ({n_copies * (base.packed.numel() + ROUTER_BYTES) / 1e9:.1f} GB)")
        self.stream = torch.cuda.current_stream()
        self.ws = {}

    def workspace(self, M):
        if M not in self.ws:
            self.ws[M] = self.B.Workspace(self.cfg, M)
        return self.ws[M]

    def event(self):
        return self.torch.cuda.Event(enable_timing=True)


def time_graph_region(ctx, graphs, runs):
    """Median over `runs` of the GPU time of replaying `graphs` (a list of
    (graph, times)) back to back, each run behind one untimed replay of the
    first graph so that the region holds GPU work only.  Returns (median ms,
    list of run ms)."""
    torch = ctx.torch
    res = []
    for _ in range(runs):
        graphs[0][0].replay()            # keeps the GPU busy while the region is enqueued
        e0, e1 = ctx.event(), ctx.event()
        e0.record(ctx.stream)
        for g, n in graphs:
            for _ in range(n):
                g.replay()
        e1.record(ctx.stream)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1))
    return float(np.median(res)), res


def measure_steps(ctx, workload, K, W, path):
    """decode / verify / stack: K timed steps replayed from graphs (after W
    warm-up steps); returns the workload's result dict."""
    torch, B, synth, shape, cfg = ctx.torch, ctx.B, ctx.synth, ctx.shape, ctx.cfg
    M = TOKENS[workload]
    stack = workload == "stack"
    n_layers = STACK_LAYERS if stack else min(ctx.args.copies, len(ctx.copies))
    chunk = max(1, min(8 if stack else ctx.args.chunk, K))
    ws = ctx.workspace(M)
    X = torch.from_numpy(synth.make_tokens(shape, 2, chunk * M).view(np.int16)).view(torch.bfloat16).cuda()
    ids = torch.empty((chunk, M, shape.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((chunk, M, shape.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((chunk, M, shape.hidden), dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty_like(out)
    xn = torch.empty_like(out)

    def step(i, s):
        x_in = X[i * M:(i + 1) * M]
        if stack:
            for l in range(n_layers):
                pk, rt = ctx.copies[l]
                bufs = (out[i], out2[i])     # layer l reads layer l-1's output
                if path == "layer":
                    if l == 0:
                        B.layer(cfg, rt, pk, x_in, ids[i], w[i], bufs[0], ws.buf)
                    else:
                        B.layer(cfg, rt, pk, bufs[(l - 1) % 2], ids[i], w[i], bufs[l % 2], ws.buf,
                                flags=B.MOE_F_INPUT_RMSNORM, x_norm=xn[i])
                elif l == 0:
                    B.route(cfg, rt, x_in, ids[i], w[i], ws.buf)
                    B.forward(cfg, pk, x_in, ids[i], w[i], bufs[0], ws.buf)
                else:
                    B.route(cfg, rt, bufs[(l - 1) % 2], ids[i], w[i], ws.buf, flags=B.MOE_F_INPUT_RMSNORM,
                            x_norm=xn[i])
                    B.forward(cfg, pk, xn[i], ids[i], w[i], bufs[l % 2], ws.buf)
        else:
            pk, rt = ctx.copies[s % n_layers]
            if path == "layer":
                B.layer(cfg, rt, pk, x_in, ids[i], w[i], out[i], ws.buf)
            else:
                B.route(cfg, rt, x_in, ids[i], w[i], ws.buf)
                B.forward(cfg, pk, x_in, ids[i], w[i], out[i], ws.buf)

    # exactly W warm-up steps, eager
    for s in range(W):
        step(s % chunk, s)
    torch.cuda.synchronize()

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                step(i, i)
        return g

    g = capture(chunk)
    graphs = [(g, K // chunk)]
    if K % chunk:
        graphs.append((capture(K % chunk), 1))
    ms, runs = time_graph_region(ctx, graphs, ctx.args.runs)
    ms_per_step = ms / K
    ids_np = ids.cpu().numpy()
    if stack:
        uniq = 8.0
        bytes_per_step = float(n_layers * step_bytes(8, 1))
    else:
        u = [len(np.unique(ids_np[i])) for i in range(chunk)]
        uniq = float(np.mean(u))
        bytes_per_step = float(np.mean([step_bytes(n, M) for n in u]))
    gbs = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    per_token = ms_per_step * 1e3 / (n_layers if stack else M)
    log(f"{workload}: {K} steps, runs {', '.join(f'{r:.3f}' for r in runs)} ms: {ms_per_step * 1e3:.2f} us/step, "
        f"{gbs:.0f} GB/s, unique experts/step {uniq:.2f}")
    return {"workload": WORKLOAD_NAMES[workload], "tokens_per_step": M, "steps": K, "warmup": W,
            "ms_per_step": ms_per_step, "run_ms": [round(r, 4) for r in runs], "gbs": gbs,
            "us_per_token": per_token, "bytes_per_step": bytes_per_step, "unique_experts_per_step": uniq,
            "resident_layer_copies": n_layers, "graph_steps_per_replay": chunk,
            "_buffers": (X, ids, w, out, ws)}


def stage_times(ctx, M, bufs, n_layers):
    """Per-launch duration of each small-M entry point on its own: a graph of n
    back-to-back launches over the same rotation of layer copies, replayed
    between HIP events on the launch stream; duration = elapsed / n."""
    torch, B, cfg = ctx.torch, ctx.B, ctx.cfg
    X, ids, w, out, ws = bufs
    chunk = ids.shape[0]
    out2 = torch.empty_like(out)
    n = max(chunk, ctx.args.stage_steps)
    names = ("route", "forward", "gate_up", "down")
    res = {}
    for stage, nm in enumerate(names):
        gs = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gs):
            for i in range(n):
                pk, rt = ctx.copies[i % n_layers]
                j = i % chunk
                x_in = X[j * M:(j + 1) * M]
                if stage == 0:
                    B.route(cfg, rt, x_in, ids[j], w[j], ws.buf)
                elif stage == 1:
                    B.forward(cfg, pk, x_in, ids[j], w[j], out2[j], ws.buf)
                elif stage == 2:
                    B.gate_up(cfg, pk, x_in, ids[j], ws.buf)
                else:
                    B.down(cfg, pk, ids[j], w[j], out2[j], ws.buf)
        gs.replay()
        torch.cuda.synchronize()
        ms, _ = time_graph_region(ctx, [(gs, 4)], 1)
        res[nm] = round(ms * 1e3 / (4 * n), 3)
        del gs
    return res


def roofline_steps(ctx, r, path):
    """Roofline of the dominant kernel of a decode/verify/stack measurement."""
    M = r["tokens_per_step"]
    stack = r["workload"] == WORKLOAD_NAMES["stack"]
    # moe_layer_w4a16 takes the one launch for M <= 2 (k_layer), the
    # separate kernels above
    one_launch = path == "layer" and M <= 2
    if one_launch:
        # k_layer is the only kernel, one launch per layer step
        launches = STACK_LAYERS if stack else 1
        us = r["ms_per_step"] * 1e3 / launches
        nbytes = r["bytes_per_step"] / launches
        kernel = "k_layer (one launch per layer: router, top-k, shared and routed experts, output)"
    else:
        # separate kernels; the dominant one is k_gate_up: the gate_up weights of
        # the step's distinct experts and of the shared expert, and the token rows
        us = r["stage_us"]["gate_up"]
        nbytes = r["unique_experts_per_step"] * EXPERT_GU_BYTES + SHARED_GU_BYTES + M * 2560 * 2
        kernel = "k_gate_up (routed INT4 gate_up + SiLU of the step's distinct experts, shared gate_up)"
    achieved = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(r["workload"]) if one_launch else None,
            "bytes_per_launch": int(nbytes), "us_per_launch": round(us, 3)}


def measure_prefill(ctx, K, W):
    """One 4096-token chunk per step: route (router GEMM + top-k) and forward
    (permutation, grouped GEMMs, combine), each timed eagerly between HIP
    events on the launch stream; and the whole step replayed from a graph."""
    torch, B, synth, shape, cfg = ctx.torch, ctx.B, ctx.synth, ctx.shape, ctx.cfg
    M = TOKENS["prefill"]
    ws = ctx.workspace(M)
    pk, rt = ctx.copies[0]
    X = torch.from_numpy(synth.make_tokens(shape, 2, M).view(np.int16)).view(torch.bfloat16).cuda()
    ids = torch.empty((M, shape.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((M, shape.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((M, shape.hidden), dtype=torch.bfloat16, device="cuda")
    for _ in range(W):
        B.route(cfg, rt, X, ids, w, ws.buf)
        B.forward(cfg, pk, X, ids, w, out, ws.buf)
    torch.cuda.synchronize()
    ev = [[ctx.event() for _ in range(3)] for _ in range(K)]
    for e in ev:
        e[0].record(ctx.stream)
        B.route(cfg, rt, X, ids, w, ws.buf)
        e[1].record(ctx.stream)
        B.forward(cfg, pk, X, ids, w, out, ws.buf)
        e[2].record(ctx.stream)
    torch.cuda.synchronize()
    t = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])] for e in ev]) * 1e3
    med = np.median(t, axis=0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.route(cfg, rt, X, ids, w, ws.buf)
        B.forward(cfg, pk, X, ids, w, out, ws.buf)
    ms, runs = time_graph_region(ctx, [(g, K)], ctx.args.runs)
    ms_per_step = ms / K
    nbytes = 512 * EXPERT_BYTES + SHARED_GU_BYTES + SHARED_DN_BYTES + ROUTER_BYTES + M * TOKEN_IO_BYTES
    flops = prefill_flops(M)
    tflops = flops / (med[1] * 1e-6) / 1e12
    log(f"prefill: route {med[0]:.1f} us, forward {med[1]:.1f} us (eager medians); graph {ms_per_step * 1e3:.1f} us/chunk")
    return {"workload": WORKLOAD_NAMES["prefill"], "tokens_per_step": M, "steps": K, "warmup": W,
            "ms_per_step": ms_per_step, "run_ms": [round(r, 4) for r in runs],
            "gbs": nbytes / (ms_per_step * 1e-3) / 1e9, "us_per_token": ms_per_step * 1e3 / M,
            "bytes_per_step": float(nbytes),
            "stage_us": {"route": round(float(med[0]), 3), "forward": round(float(med[1]), 3)},
            "roofline": {"bound": "mfma", "kernel": "moe_forward_w4a16 at M=4096 (grouped GEMM kernels + permutation "
                                                      "+ combine)", "achieved": round(tflops, 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic(WORKLOAD_NAMES["prefill"]), "flops_per_launch": flops}}


def measure_lmhead(ctx, K, W, fp8):
    """The LM head for one token (M = 1): the BF16 head 157,184 x 2,560, or
    its FP8 copy (quantised once on the device, outside the timed region);
    K products replayed from graphs of 32."""
    torch, B, synth = ctx.torch, ctx.B, ctx.synth
    V, H = synth.LM_VOCAB, LM_HIDDEN
    if getattr(ctx, "lm", None) is None:
        t0 = time.time()
        wb = torch.from_numpy(synth.make_lmhead(V, H, 1, threads=16).view(np.int16)).cuda()
        q = torch.empty((V, H), dtype=torch.uint8, device="cuda")
        sc = torch.empty(V, dtype=torch.float32, device="cuda")
        B.lmhead_quantize_fp8(wb, q, sc)
        torch.cuda.synchronize()
        ctx.lm = (wb, q, sc)
        log(f"LM head generated and quantised in {time.time() - t0:.1f}s")
    wb, q, sc = ctx.lm
    x = torch.from_numpy(synth.make_tokens(ctx.shape, 3, 1).view(np.int16)).cuda()
    out = torch.empty((1, V), dtype=torch.float32, device="cuda")

    def call():
        if fp8:
            B.lmhead_fp8(q, sc, x, out)
        else:
            B.lmhead_bf16(wb, x, out)

    for _ in range(W):
        call()
    torch.cuda.synchronize()
    G = 32
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(G):
            call()
    reps = max(1, K // G)
    ms, runs = time_graph_region(ctx, [(g, reps)], ctx.args.runs)
    ms_per_step = ms / (reps * G)
    nbytes = V * H * (1 if fp8 else 2) + (V * 4 if fp8 else 0) + H * 2 + V * 4
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    name = "lmhead_fp8" if fp8 else "lmhead_bf16"
    log(f"{name}: {reps * G} products, {ms_per_step * 1e3:.2f} us each, {gbs:.0f} GB/s")
    return {"workload": WORKLOAD_NAMES[name], "tokens_per_step": 1, "steps": reps * G, "warmup": W,
            "ms_per_step": ms_per_step, "run_ms": [round(r, 4) for r in runs], "gbs": gbs,
            "us_per_token": ms_per_step * 1e3, "bytes_per_step": float(nbytes),
            "roofline": {"bound": "hbm", "kernel": f"k_lmhead_gemv<{'fp8' if fp8 else 'bf16'}> ({V} x {H})",
                         "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "bytes_per_launch": nbytes,
                         "us_per_launch": round(ms_per_step * 1e3, 3)}}


def measure_fmt(ctx, wl, K, W):
    """Decode (M = 1) with the routed experts in MXFP4 or block FP8, rotating
    over FMT_COPIES resident copies of the layer (experts, shared expert and
    router; copy c has the router of layer seed 1000 + c), replayed from
    graphs of 64 steps.  MXFP4: one moe_layer_mxfp4 launch per step on the
    tiled layout, with the two-call path (moe_route + moe_forward_fmt on the
    plain layout) timed beside it; block FP8: the two-call path."""
    torch, B, synth, shape = ctx.torch, ctx.B, ctx.synth, ctx.shape
    fmt = synth.FMT_MXFP4 if wl == "decode_mxfp4" else synth.FMT_FP8_BLOCK
    t0 = time.time()
    src = synth.make_layer_fmt(shape, 1, fmt, threads=16)
    base = B.FmtLayerDev(src)
    copies = [base]
    for c in range(1, FMT_COPIES):
        d = B.FmtLayerDev.__new__(B.FmtLayerDev)
        d.shape, d.fmt, d.cfg = base.shape, base.fmt, base.cfg
        for name in ("w13_q", "w13_s", "w2_q", "w2_s", "sh_w13", "sh_w2"):
            setattr(d, name, getattr(base, name).clone())
        d.weights = B.MoeWeightsFmt(*(B._ptr(getattr(d, n)) for n in ("w13_q", "w13_s", "w2_q", "w2_s",
                                                                      "sh_w13", "sh_w2")))
        copies.append(d)
    for c, d in enumerate(copies):
        d.router_w = torch.from_numpy(synth.make_router(shape, 1000 + c)).cuda()
    packed = []
    if fmt == synth.FMT_MXFP4:
        mx = B.MxLayerDev(src)
        packed = [mx.packed] + [mx.packed.clone() for _ in range(1, FMT_COPIES)]
    torch.cuda.synchronize()
    log(f"{wl}: {FMT_COPIES} copies resident in {time.time() - t0:.1f}s")
    ws = ctx.workspace(1)
    X = torch.from_numpy(synth.make_tokens(shape, 2, 64).view(np.int16)).view(torch.bfloat16).cuda()
    ids = torch.empty((1, shape.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, shape.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((1, shape.hidden), dtype=torch.bfloat16, device="cuda")

    def step_calls(i):
        d = copies[i % FMT_COPIES]
        x = X[i % 64:i % 64 + 1]
        B.route(d.cfg, d.router_w, x, ids, w, ws.buf)
        B.forward_fmt(d, x, ids, w, out, ws.buf)

    def step_one(i):
        d = copies[i % FMT_COPIES]
        B.layer_mxfp4(d.cfg, d.router_w, packed[i % FMT_COPIES], X[i % 64:i % 64 + 1], ids, w, out, ws.buf)

    G = 64
    reps = max(1, K // G)

    def timed(step):
        for i in range(W):
            step(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(G):
                step(i)
        ms, runs = time_graph_region(ctx, [(g, reps)], ctx.args.runs)
        return ms / (reps * G), runs

    ms_calls, runs_calls = timed(step_calls)
    one = fmt == synth.FMT_MXFP4
    ms_per_step, runs = timed(step_one) if one else (ms_calls, runs_calls)
    nbytes = 8 * EXPERT_BYTES_FMT[wl] + SHARED_GU_BYTES + SHARED_DN_BYTES + ROUTER_BYTES + TOKEN_IO_BYTES
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    log(f"{wl}: {reps * G} steps, {ms_per_step * 1e3:.2f} us/step, {gbs:.0f} GB/s"
        + (f" (one launch; two calls {ms_calls * 1e3:.2f} us/step)" if one else ""))
    kernel = ("moe_layer_mxfp4 (k_layer, MXFP4 routed experts, one launch)" if one
              else "moe_route + moe_forward_fmt (k_route, k_fmt_gate_up, k_fmt_down)")
    return {"workload": WORKLOAD_NAMES[wl], "tokens_per_step": 1, "steps": reps * G, "warmup": W,
            "ms_per_step": ms_per_step, "run_ms": [round(r, 4) for r in runs], "gbs": gbs,
            "us_per_token": ms_per_step * 1e3, "bytes_per_step": float(nbytes), "resident_layer_copies": FMT_COPIES,
            "us_per_token_two_calls": round(ms_calls * 1e3, 3),
            "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic(WORKLOAD_NAMES[wl]) if one else None,
                         "bytes_per_launch": nbytes, "us_per_launch": round(ms_per_step * 1e3, 3)}}


def measure_mtp(ctx, K, W):
    """The speculative-decoding round on the 40-layer stack (mtp.MtpRound):
    3 draft steps of a draft layer (M = 1 each) and a 4-position verify
    through the 40 layers; beside it the verify alone and one decode token
    through the same 40 layers (M = 1), each replayed from graphs."""
    torch, B, synth, shape, cfg = ctx.torch, ctx.B, ctx.synth, ctx.shape, ctx.cfg
    from w4a16_grouped_quantized_amd.mtp import MtpRound
    stack = [ctx.copies[l] for l in range(STACK_LAYERS)]
    stack = [(rt, pk) for pk, rt in stack]
    draft = (ctx.copies[STACK_LAYERS][1], ctx.copies[STACK_LAYERS][0])
    ws = ctx.workspace(4)
    r = MtpRound(cfg, stack, draft, ws)
    X = torch.from_numpy(synth.make_tokens(shape, 5, 1).view(np.int16)).view(torch.bfloat16).cuda()
    r.rows[0:1].copy_(X)
    # unique experts per verify layer (for the verify's bytes)
    uniq = []
    r.round(record_verify=lambda l, xn, ids, w, out: uniq.append(len(set(ids.cpu().numpy().ravel().tolist()))))
    for _ in range(W):
        r.round()
    torch.cuda.synchronize()
    # decode: one token through the same layers, RMSNorm between them
    ids1 = torch.empty((1, shape.top_k), dtype=torch.int32, device="cuda")
    w1 = torch.empty((1, shape.top_k), dtype=torch.float32, device="cuda")
    b1 = (torch.empty((1, shape.hidden), dtype=torch.bfloat16, device="cuda"),
          torch.empty((1, shape.hidden), dtype=torch.bfloat16, device="cuda"))
    xn1 = torch.empty((1, shape.hidden), dtype=torch.bfloat16, device="cuda")
    ws1 = ctx.workspace(1)

    def decode():
        for l, (rt, pk) in enumerate(stack):
            if l == 0:
                B.layer(cfg, rt, pk, X, ids1, w1, b1[0], ws1.buf)
            else:
                B.layer(cfg, rt, pk, b1[(l - 1) % 2], ids1, w1, b1[l % 2], ws1.buf, flags=B.MOE_F_INPUT_RMSNORM,
                        x_norm=xn1)

    graphs = {}
    for name, fn in (("round", r.round), ("verify", r.verify), ("drafts", r.drafts), ("decode", decode)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs[name] = g
    t = {}
    runs_round = None
    for name, g in graphs.items():
        ms, runs = time_graph_region(ctx, [(g, K)], ctx.args.runs)
        t[name] = ms / K * 1e3
        if name == "round":
            runs_round = runs
    ratio = t["verify"] / t["decode"]
    vbytes = sum(step_bytes(u, 4) for u in uniq)
    gbs = vbytes / (t["verify"] * 1e-6) / 1e9
    log(f"mtp_round: {t['round']:.1f} us/round (drafts {t['drafts']:.1f}, verify {t['verify']:.1f}); decode through "
        f"{STACK_LAYERS} layers {t['decode']:.1f} us; verify:decode {ratio:.2f}; unique experts per verify layer "
        f"{np.mean(uniq):.2f}")
    return {"workload": WORKLOAD_NAMES["mtp_round"], "tokens_per_step": 4, "steps": K, "warmup": W,
            "ms_per_step": t["round"] / 1e3, "run_ms": [round(x, 4) for x in runs_round],
            "gbs": gbs, "us_per_token": t["round"] / MTP_ACCEPT, "bytes_per_step": float(vbytes),
            "us_per_round": round(t["round"], 3), "us_drafts": round(t["drafts"], 3),
            "us_verify": round(t["verify"], 3), "us_decode_stack": round(t["decode"], 3),
            "verify_to_decode": round(ratio, 3), "pages_verify_to_decode": 2.26,
            "unique_experts_per_verify_layer": round(float(np.mean(uniq)), 2),
            "tokens_per_s_at_accept": {str(a): round(a / (t["round"] * 1e-6), 1) for a in (1.0, 2.0, 3.0, MTP_ACCEPT, 4.0)},
            "roofline": {"bound": "hbm", "kernel": "verify step: 40 layers at M = 4 (moe_route + moe_forward_w4a16 "
                                                   "per layer)", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                         "bytes_per_launch": vbytes, "us_per_launch": round(t["verify"], 3)}}


def read_ceiling(ctx, gib=2, runs=5):
    """GB/s of the plain streaming read (moe_probe_read) over a buffer far
    larger than the last-level cache: median of `runs`."""
    torch, B = ctx.torch, ctx.B
    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(3)
    blocks = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    B.probe_read(buf, sink, blocks)
    torch.cuda.synchronize()
    res = []
    for _ in range(runs):
        e0, e1 = ctx.event(), ctx.event()
        e0.record(ctx.stream)
        B.probe_read(buf, sink, blocks)
        e1.record(ctx.stream)
        torch.cuda.synchronize()
        res.append(n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    gbs = float(np.median(res))
    log(f"read ceiling: {gbs:.0f} GB/s ({gib} GiB, 10 KB tiles per wavefront, {blocks} workgroups; runs "
        f"{', '.join(f'{r:.0f}' for r in res)})")
    return {"gbs": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4), "bytes": n,
            "kernel": "moe_probe_read (10 KB tiles per wavefront, double-buffered 16-byte non-temporal loads, every byte once)"}


def summary(r, ceiling):
    d = {k: v for k, v in r.items() if not k.startswith("_")}
    for k in ("ms_per_step", "gbs", "us_per_token"):
        d[k] = round(d[k], 6 if k == "ms_per_step" else 3)
    if ceiling and d.get("roofline", {}).get("unit") == "GB/s":
        d["roofline"]["frac_of_read_ceiling"] = round(d["roofline"]["achieved"] / ceiling["gbs"], 4)
    return d


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(expert and tensor sharding are design notes only); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    from w4a16_grouped_quantized_amd import binding as B
    B.lib()

    head = args.workload
    extras = [] if (args.no_extras or head != "decode") else ["verify2", "verify4", "stack", "prefill",
                                                                "lmhead_fp8", "lmhead_bf16", "decode_mxfp4",
                                                                "decode_fp8block", "mtp_round"]
    need = 1 if head in ("prefill", "lmhead_fp8", "lmhead_bf16", "decode_mxfp4", "decode_fp8block") else args.copies
    if head == "stack" or "stack" in extras:
        need = max(need, STACK_LAYERS)
    if head == "mtp_round" or "mtp_round" in extras:
        need = max(need, STACK_LAYERS + 1)
    ctx = Ctx(args, need)

    results = {}
    for wl in [head] + extras:
        K, W = (args.steps, args.warmup) if wl == head else EXTRA_STEPS[wl]
        if wl == "prefill":
            results[wl] = measure_prefill(ctx, K, W)
            continue
        if wl in ("lmhead_fp8", "lmhead_bf16"):
            results[wl] = measure_lmhead(ctx, K, W, wl == "lmhead_fp8")
            continue
        if wl in ("decode_mxfp4", "decode_fp8block"):
            results[wl] = measure_fmt(ctx, wl, K, W)
            continue
        if wl == "mtp_round":
            results[wl] = measure_mtp(ctx, K, W)
            continue
        r = measure_steps(ctx, wl, K, W, args.path)
        if TOKENS[wl] > 1 or args.path == "calls" or wl == head:
            r["stage_us"] = stage_times(ctx, TOKENS[wl], r["_buffers"], min(args.copies, len(ctx.copies)))
            log(f"{wl}: entry point us per launch (graphs of back-to-back launches): " +
                " ".join(f"{k} {v:.2f}" for k, v in r["stage_us"].items()))
        r["roofline"] = roofline_steps(ctx, r, args.path)
        results[wl] = r

    ceiling = read_ceiling(ctx)

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy: {args.calib_copy_mib} MiB x 2")

    cpu = None
    if not args.no_cpu_baseline and head in ("decode", "verify2", "verify4", "stack"):
        cpu = cpu_baseline(ctx.shape, ctx.layer, args.cpu_baseline_seconds)

    h = summary(results[head], ceiling)
    line = {
        "metric": "MoE layer us/token and achieved HBM GB/s at batch 1 (W4A16 g32, top-8 of 512)",
        "value": round(h["gbs"], 1),
        "unit": "GB/s",
        "us_per_token": h["us_per_token"],
        "n_gpus": 1,
        "steps": h["steps"],
        "warmup": h["warmup"],
        "ms_per_step": h["ms_per_step"],
        "run_ms": h["run_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": h["workload"],
            "hidden": 2560, "n_experts": 512, "top_k": 8, "moe_intermediate": 768, "group_size": 32,
            "tokens_per_step": h["tokens_per_step"], "resident_layer_copies": h.get("resident_layer_copies", 1),
            "graph_steps_per_replay": h.get("graph_steps_per_replay", 1), "timed_runs": args.runs,
            "algorithmic_bytes_per_step": int(h["bytes_per_step"]),
            "unique_experts_per_step": h.get("unique_experts_per_step", 512.0),
            "compute": "bf16 activations, int4 weights, fp32 accumulate",
        },
        "stage_us": h.get("stage_us"),
        "roofline": h["roofline"],
        "read_ceiling": ceiling,
        "cpu_baseline": cpu,
        "extra": {wl: summary(results[wl], ceiling) for wl in extras},
        "build": ctx.B.build_info(),
    }
    print(json.dumps(line), flush=True)


DIGEST_EXCLUDED = ("probe.hip",)


def kernel_sources_digest() -> str:
    """sha256 over the code of the layer's HIP sources (comments and blank
    lines stripped, see source_code_only); a measured traffic figure is valid
    only for the code it was measured on.  The read-rate probe (probe.hip) is
    a measurement aid that no layer kernel includes, so it is left out."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4a16_grouped_quantized_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")) and name not in DIGEST_EXCLUDED:
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                h.update(name.encode() + b"\0" + source_code_only(f.read()).encode())
    return h.hexdigest()


def source_code_only(text: str) -> str:
    """C++ source without its comments, trailing blanks and empty lines:
    string and character literals are kept whole (a // or /* inside one is
    not a comment)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    lines = ("".join(out)).split("\n")
    return "\n".join(l.rstrip() for l in lines if l.strip())


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed counter
    profile (profiles/<workload>_traffic.txt), or None when there is none or
    the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("sources_sha256") != kernel_sources_digest():
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def oracle_tokens_per_time(shape, layer, x, seconds):
    """Route + forward of single decode tokens through the oracle for about
    `seconds` (after one warm-up token); returns (tokens, elapsed s)."""
    from oracle import oracle as O
    ids, w, _, _ = O.route(shape, layer.router_w, x[:1])
    O.forward(shape, layer, x[:1], ids, w)
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds and n < x.shape[0] - 1:
        xt = x[1 + n:2 + n]
        ids, w, _, _ = O.route(shape, layer.router_w, xt)
        O.forward(shape, layer, xt, ids, w)
        n += 1
    return n, time.perf_counter() - t0


def cpu_baseline(shape, layer, seconds):
    """The oracle (fp64, plain loops) on the host: route + forward for as many
    decode tokens of the same layer as fit in about `seconds`, on all of the
    threads OpenMP gives it here, and again in a child process on one thread."""
    from oracle import oracle as O
    from w4a16_grouped_quantized_amd import synth
    O.lib()
    threads = O.num_threads()
    x = synth.make_tokens(shape, 2, 4096)
    n, dt = oracle_tokens_per_time(shape, layer, x, seconds)
    us = dt / n * 1e6
    log(f"cpu baseline (oracle): {n} tokens in {dt:.1f}s, {us:.0f} us/token, {threads} threads")
    one = None
    try:
        env = dict(os.environ, OMP_NUM_THREADS="1")
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-one-core", str(seconds / 2)],
                           env=env, capture_output=True, text=True, timeout=600)
        if r.returncode == 0:
            one = json.loads(r.stdout.strip().splitlines()[-1])
            log(f"cpu baseline (oracle, 1 thread): {one['tokens']} tokens, {one['us_per_token']:.0f} us/token")
        else:
            log(f"one-thread oracle run failed: {r.stderr[-300:]}")
    except (subprocess.SubprocessError, ValueError) as e:
        log(f"one-thread oracle run failed: {e}")
    res = {"value": round(step_bytes(8, 1) / (us * 1e-6) / 1e9, 4), "unit": "GB/s", "us_per_token": round(us, 1),
           "cores": threads, "kind": "oracle",
           "sample": f"{n} decode tokens (M=1) of the seed-1 Ling-shape layer, route + forward"}
    if one:
        res["one_core"] = {"value": round(step_bytes(8, 1) / (one["us_per_token"] * 1e-6) / 1e9, 4), "unit": "GB/s",
                           "us_per_token": round(one["us_per_token"], 1), "cores": 1,
                           "sample": f"{one['tokens']} decode tokens, same layer"}
    return res


def oracle_one_core(seconds):
    """Child process of cpu_baseline: the oracle with OMP_NUM_THREADS=1."""
    from oracle import oracle as O
    from w4a16_grouped_quantized_amd import synth
    O.lib()
    layer = synth.make_layer(synth.LING, 1, threads=16)
    x = synth.make_tokens(synth.LING, 2, 4096)
    n, dt = oracle_tokens_per_time(synth.LING, layer, x, seconds)
    print(json.dumps({"tokens": n, "us_per_token": dt / n * 1e6, "threads": O.num_threads()}), flush=True)


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--oracle-one-core":
        oracle_one_core(float(sys.argv[2]))
    else:
        main()
