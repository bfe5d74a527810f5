#!/usr/bin/env python3
"""Benchmark of the W4A16 grouped-quantized MoE layer on one MI355X.

Default workload (one "step" = one decode token through one Ling-shape MoE
layer: route + gate_up/SiLU + down + weighted combine + shared expert, M = 1):
  hidden 2560, 512 routed experts, top-8, moe_intermediate 768, INT4 g32
  routed experts with bf16 scales, bf16 shared expert, fp32 router.
Steps rotate over C resident copies of the layer (distinct device memory,
distinct seeded routers), so a step never finds its weights in the 256 MB
last-level cache; the step chain is captured once in a HIP graph and
replayed.  Throughput is algorithmic bytes per step / time (GB/s) and
microseconds per token.

Other workloads (for measurement runs; the default is the one reported):
  --workload verify2 / verify4   M = 2 / 4 tokens per step (speculative verify)
  --workload stack               one token through 40 stacked layers with
                                 RMSNorm between them (one step = 40 layers)
  --workload prefill             one chunk of M = 4096 tokens per step (router
                                 GEMM, grouped expert GEMMs on the matrix cores)

Prints one JSON line.
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

PEAK_HBM_GBS = 8000.0

# Algorithmic bytes (Ling shape): every weight byte a step must read once,
# plus activations in and out.
EXPERT_GU_BYTES = 2 * 768 * 2560 // 2 + 2 * 768 * (2560 // 32) * 2     # 2,211,840
EXPERT_DN_BYTES = 2560 * 768 // 2 + 2560 * (768 // 32) * 2             # 1,105,920
EXPERT_BYTES = EXPERT_GU_BYTES + EXPERT_DN_BYTES                        # 3,317,760
SHARED_GU_BYTES = 2 * 768 * 2560 * 2                                    # 7,864,320
SHARED_DN_BYTES = 2560 * 768 * 2                                        # 3,932,160
ROUTER_BYTES = 512 * 2560 * 4                                           # 5,242,880
TOKEN_IO_BYTES = 2 * 2560 * 2                                           # x in, out back


WORKLOAD_NAMES = {"decode": "ling_moe_layer_decode_m1", "verify2": "ling_moe_layer_verify_m2",
                  "verify4": "ling_moe_layer_verify_m4", "stack": "ling_moe_stack40_decode_m1",
                  "prefill": "ling_moe_layer_prefill_m4096"}


def step_bytes(n_unique_experts: int, M: int) -> int:
    return n_unique_experts * EXPERT_BYTES + SHARED_GU_BYTES + SHARED_DN_BYTES + ROUTER_BYTES + M * TOKEN_IO_BYTES


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=4096)
    p.add_argument("--warmup", type=int, default=512)
    p.add_argument("--workload", default="decode", choices=["decode", "verify2", "verify4", "stack", "prefill"])
    p.add_argument("--copies", type=int, default=None,
                   help="resident layer copies to rotate over (default 32; 1 for prefill, which reads every expert)")
    p.add_argument("--chunk", type=int, default=256, help="steps captured per graph")
    p.add_argument("--path", default="layer", choices=["layer", "calls"],
                   help="layer: one moe_layer_w4a16 call per layer step (one launch at small M); "
                        "calls: moe_route then moe_forward_w4a16")
    p.add_argument("--cpu-baseline-seconds", type=float, default=12.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--stage-steps", type=int, default=256, help="eager steps timed per stage")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="after timing, run a plain device copy of this many MiB (reference for HBM byte counters)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(expert and tensor sharding are design notes only); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from w4a16_grouped_quantized_amd import binding as B
    from w4a16_grouped_quantized_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    B.lib()
    shape = synth.LING
    cfg = B.config(shape)
    M = {"decode": 1, "verify2": 2, "verify4": 4, "stack": 1, "prefill": 4096}[args.workload]
    prefill = args.workload == "prefill"
    if args.copies is None:
        args.copies = 1 if prefill else 32
    if prefill:
        args.chunk = min(args.chunk, 4)
    n_layers = 40 if args.workload == "stack" else args.copies

    t0 = time.time()
    layer = synth.make_layer(shape, 1, threads=16)
    base = B.MoeLayer(layer)
    log(f"layer generated and packed in {time.time() - t0:.1f}s; build: {B.build_info()}")

    # C copies: distinct device memory; distinct seeded routers (layer seeds 1000 + c).
    copies = []
    for c in range(n_layers):
        packed = base.packed if c == 0 else base.packed.clone()
        router = torch.from_numpy(synth.make_router(shape, 1000 + c)).cuda()
        copies.append((packed, router))
    torch.cuda.synchronize()
    log(f"{n_layers} resident copies ({n_layers * (base.packed.numel() + 5242880) / 1e9:.1f} GB)")

    ws = B.Workspace(cfg, max(M, 1))
    stream = torch.cuda.current_stream()
    chunk = max(1, min(args.chunk, args.steps))
    n_tok = chunk * M
    X = torch.from_numpy(synth.make_tokens(shape, 2, n_tok).view(np.int16)).view(torch.bfloat16).cuda()
    ids = torch.empty((chunk, M, shape.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((chunk, M, shape.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((chunk, M, shape.hidden), dtype=torch.bfloat16, device="cuda")
    xn = torch.empty((chunk, M, shape.hidden), dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty((chunk, M, shape.hidden), dtype=torch.bfloat16, device="cuda")

    def run_steps(lo, hi, step_offset):
        """Enqueue steps lo..hi-1 (the graph body)."""
        for i in range(lo, hi):
            s = step_offset + i
            if args.workload == "stack":
                # one token through all layers; layer l reads the previous output
                x_in = X[i * M:(i + 1) * M]
                for l in range(n_layers):
                    pk, rt = copies[l]
                    if args.path == "layer":
                        # outputs alternate between two buffers: layer l reads layer l-1's
                        bufs = (out[i], out2[i])
                        if l == 0:
                            B.layer(cfg, rt, pk, x_in, ids[i], w[i], bufs[0], ws.buf)
                        else:
                            B.layer(cfg, rt, pk, bufs[(l - 1) % 2], ids[i], w[i], bufs[l % 2], ws.buf,
                                    flags=B.MOE_F_INPUT_RMSNORM, x_norm=xn[i])
                    elif l == 0:
                        B.route(cfg, rt, x_in, ids[i], w[i], ws.buf)
                        B.forward(cfg, pk, x_in, ids[i], w[i], out[i], ws.buf)
                    else:
                        B.route(cfg, rt, out[i], ids[i], w[i], ws.buf, flags=B.MOE_F_INPUT_RMSNORM, x_norm=xn[i])
                        B.forward(cfg, pk, xn[i], ids[i], w[i], out[i], ws.buf)
            else:
                pk, rt = copies[s % n_layers]
                x_in = X[i * M:(i + 1) * M]
                if args.path == "layer":
                    B.layer(cfg, rt, pk, x_in, ids[i], w[i], out[i], ws.buf)
                else:
                    B.route(cfg, rt, x_in, ids[i], w[i], ws.buf)
                    B.forward(cfg, pk, x_in, ids[i], w[i], out[i], ws.buf)

    # warm the stream outside capture, then capture one chunk
    run_steps(0, chunk, 0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_steps(0, chunk, 0)
    reps = max(1, args.steps // chunk)
    steps = reps * chunk
    wreps = max(1, args.warmup // chunk)
    for _ in range(wreps):
        g.replay()
    torch.cuda.synchronize()

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    tw = time.perf_counter()
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - tw
    ms = e0.elapsed_time(e1)
    ms_per_step = ms / steps

    ids_np = ids.cpu().numpy()
    if args.workload == "stack":
        uniq = 8.0  # per layer at M = 1
        bytes_per_step = n_layers * step_bytes(8, 1)
    else:
        uniq = float(np.mean([len(np.unique(ids_np[i])) for i in range(chunk)]))
        bytes_per_step = float(np.mean([step_bytes(len(np.unique(ids_np[i])), M) for i in range(chunk)]))
    gbs = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    log(f"{steps} steps in {ms:.2f} ms (wall {wall * 1e3:.2f} ms): {ms_per_step * 1e3:.2f} us/step, "
        f"{gbs:.0f} GB/s, unique experts/step {uniq:.2f}")

    one_launch = False
    if prefill:
        # route (router GEMM + top-k) and forward (permutation, grouped GEMMs,
        # combine) timed separately, eager, HIP events on the launch stream
        def time_calls(n):
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
            for i in range(n):
                pk, rt = copies[i % n_layers]
                j = i % chunk
                x_in = X[j * M:(j + 1) * M]
                e = ev[i]
                e[0].record(stream)
                B.route(cfg, rt, x_in, ids[j], w[j], ws.buf)
                e[1].record(stream)
                B.forward(cfg, pk, x_in, ids[j], w[j], out[j], ws.buf)
                e[2].record(stream)
            torch.cuda.synchronize()
            r = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])] for e in ev]) * 1e3
            return np.median(r, axis=0), np.mean(r, axis=0)

        time_calls(2)
        st_med, st_mean = time_calls(max(4, min(args.stage_steps, 16)))
        log(f"call us (median) route {st_med[0]:.1f} forward {st_med[1]:.1f}; (mean) {st_mean[0]:.1f} {st_mean[1]:.1f}")
        pairs = M * shape.top_k
        flops = 2.0 * pairs * (2 * 768 * 2560 + 2560 * 768) + 2.0 * M * (2 * 768 * 2560 + 2560 * 768)
        tflops = flops / (st_mean[1] * 1e-6) / 1e12
        stage = {"route": round(float(st_mean[0]), 3), "forward": round(float(st_mean[1]), 3)}
        roof = {"bound": "mfma", "kernel": "moe_forward_w4a16 at M=4096 (grouped GEMM kernels + permutation + combine)",
                "achieved": round(tflops, 2), "peak": 2500.0, "unit": "TFLOP/s", "frac": round(tflops / 2500.0, 4),
                "traffic": None, "flops_per_launch": flops}
    else:
        # Per-entry-point durations, each a graph of n back-to-back launches of
        # that call alone over the same rotation of layer copies, replayed
        # between HIP events on the launch stream; duration per launch =
        # elapsed / n.  route = moe_route (k_route), forward = moe_forward_w4a16
        # on the routed ids (k_gate_up then k_down), and those two kernels
        # alone.
        stage_names = ("route", "forward", "gate_up", "down")

        def stage_graph(stage, n):
            gs = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gs):
                for i in range(n):
                    pk, rt = copies[i % n_layers]
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
            return gs

        def time_stages(n):
            res = []
            for stage in range(len(stage_names)):
                gs = stage_graph(stage, n)
                gs.replay()
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                reps_s = 4
                e0.record(stream)
                for _ in range(reps_s):
                    gs.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                res.append(e0.elapsed_time(e1) * 1e3 / (reps_s * n))
                del gs
            return np.array(res)

        st = time_stages(max(chunk, args.stage_steps))
        log("entry point us per launch (graph of back-to-back launches): " +
            " ".join(f"{nm} {v:.2f}" for nm, v in zip(stage_names, st)))
        stage = {nm: round(float(v), 3) for nm, v in zip(stage_names, st)}
        n_uniq = uniq if args.workload != "stack" else 8
        one_launch = args.path == "layer" and M == 1
        if one_launch:
            # the dominant kernel is the only one: k_layer, one launch per
            # layer; its duration per launch is the timed region / launches
            launches = n_layers if args.workload == "stack" else 1
            us_launch = ms_per_step * 1e3 / launches
            bytes_launch = bytes_per_step / launches
            kernel = "k_layer (one launch per layer: router, top-k, shared and routed experts, output)"
        else:
            # separate kernels (k_route, k_gate_up, k_down); the dominant one
            # is k_gate_up: the gate_up weights of the step's distinct experts
            # and of the shared expert, and the step's token rows
            us_launch = float(st[2])
            bytes_launch = n_uniq * EXPERT_GU_BYTES + SHARED_GU_BYTES + M * 2560 * 2
            kernel = "k_gate_up (routed INT4 gate_up + SiLU of the step's distinct experts, shared gate_up)"
        achieved = bytes_launch / (us_launch * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                "bytes_per_launch": int(bytes_launch), "us_per_launch": round(us_launch, 3)}

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy: {args.calib_copy_mib} MiB x 2")

    if roof.get("traffic") is None:
        roof["traffic"] = measured_traffic(WORKLOAD_NAMES[args.workload]) if one_launch or prefill else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(shape, layer, args.cpu_baseline_seconds)

    dtype = "bf16 activations, int4 weights, fp32 accumulate"
    line = {
        "metric": "MoE layer us/token and achieved HBM GB/s at batch 1 (W4A16 g32, top-8 of 512)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        # per token per layer
        "us_per_token": round(ms_per_step * 1e3 / (M if args.workload != "stack" else n_layers), 3),
        "n_gpus": 1,
        "steps": steps,
        "warmup": wreps * chunk,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[args.workload],
            "hidden": 2560, "n_experts": 512, "top_k": 8, "moe_intermediate": 768, "group_size": 32,
            "tokens_per_step": M, "resident_layer_copies": n_layers, "graph_steps_per_replay": chunk,
            "algorithmic_bytes_per_step": int(bytes_per_step), "unique_experts_per_step": uniq,
            "compute": dtype,
        },
        "stage_us": stage,
        "roofline": roof,
        "cpu_baseline": cpu,
        "build": B.build_info(),
    }
    print(json.dumps(line), flush=True)


def kernel_sources_digest() -> str:
    """sha256 over the HIP sources; a measured traffic figure is valid only
    for the sources it was measured on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4a16_grouped_quantized_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


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


def cpu_baseline(shape, layer, seconds):
    """The oracle (fp64, plain loops) on host cores: route + forward for as
    many decode tokens of the same layer as fit in about `seconds`."""
    from oracle import oracle as O
    O.lib()
    threads = O.num_threads()
    from w4a16_grouped_quantized_amd import synth
    x = synth.make_tokens(shape, 2, 4096)
    # warm-up token
    ids, w, _, _ = O.route(shape, layer.router_w, x[:1])
    O.forward(shape, layer, x[:1], ids, w)
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds and n < x.shape[0] - 1:
        xt = x[1 + n:2 + n]
        ids, w, _, _ = O.route(shape, layer.router_w, xt)
        O.forward(shape, layer, xt, ids, w)
        n += 1
    dt = time.perf_counter() - t0
    us = dt / n * 1e6
    gbs = step_bytes(8, 1) / (us * 1e-6) / 1e9
    log(f"cpu baseline (oracle): {n} tokens in {dt:.1f}s, {us:.0f} us/token, {threads} threads")
    return {"value": round(gbs, 4), "unit": "GB/s", "us_per_token": round(us, 1), "cores": threads,
            "kind": "oracle", "sample": f"{n} decode tokens (M=1) of the seed-1 Ling-shape layer, route + forward"}


if __name__ == "__main__":
    main()
