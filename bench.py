#!/usr/bin/env python3
"""Decode benchmark of the fused reconstruct-and-project linear on one MI355X.

Workload: one Gemma-3-1B-shaped decoder layer at decode, T = 1 token, rank r
(default 32): fused Q/K/V 1152 -> 1024 + 256 + 256, O 1024 -> 1152, fused MLP
gate/up 1152 -> 6912, GELU-tanh, down 6912 -> 1152. A step is one pass of that
layer (three library calls: wl_qkv_fused, wl_linear, wl_mlp_fused). Steps cycle
over 26 resident layers with their own W0 (the passthrough point, one W0 per
layer), so the 1.4 GB weight set is streamed from HBM rather than served from
the 256 MB last-level cache. Inputs are seeded synthetic draws with the value
distributions W0 ~ N(0, 0.02), s ~ 1 + N(0, 0.01), U, V ~ N(0, 0.01),
x ~ N(0, 1), already resident on the GPU when timing starts.

Prints one JSON line: tokens/s per layer (value), the roofline record of the
dominant operation (the fused MLP, about 86 % of a layer's bytes) measured with
HIP events on the launch stream during the timed region, and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
if REPO not in sys.path:
    sys.path.insert(0, REPO)

HBM_PEAK_GBS = 8000.0
METRIC = "tokens/s + achieved HBM GB/s (T=1) / MFMA TFLOP/s (T=2048) per rank"


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2600)
    p.add_argument("--warmup", type=int, default=260)
    p.add_argument("--rank", type=int, default=32)
    p.add_argument("--layers", type=int, default=26, help="distinct resident layers cycled through")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle sample budget (0 skips it)")
    return p.parse_args()


def theta_bytes(th: dict) -> int:
    """W0 + s + U + V bytes of one theta."""
    d_in, d_out, r = th["d_in"], th["d_out"], th["r"]
    return 2 * d_out * d_in + (4 * d_out if th.get("s") is not None else 0) + 2 * r * (d_out + d_in)


def main() -> int:
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path is single-device; sharding is described in DESIGN.md)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from linear_02_amd import build as wl_build
    if not os.path.exists(wl_build.LIBRARY):
        wl_build.build()
    from linear_02_amd import inputs, wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dims = inputs.GEMMA3_1B
    r, L, T = args.rank, args.layers, 1
    gen = torch.Generator().manual_seed(0)

    # Resident layers (device) and the host copy of layer 0 for the oracle.
    t_gen = time.perf_counter()
    layers_dev, acts_dev = [], []
    host_layer0 = host_acts0 = None
    for l in range(L):
        lay = inputs.layer(gen, dims, r)
        acts = inputs.layer_inputs(gen, dims, T)
        if l == 0:
            host_layer0, host_acts0 = lay, acts
        layers_dev.append({f: wl.theta_to(lay[f], dev) for f in inputs.FAMILIES})
        acts_dev.append({k: v.to(dev) for k, v in acts.items()})
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    width_qkv = dims["q"] + 2 * dims["kv"]
    y_qkv = torch.empty(T, width_qkv, dtype=torch.bfloat16, device=dev)
    y_o = torch.empty(T, dims["d_model"], dtype=torch.bfloat16, device=dev)
    y_mlp = torch.empty(T, dims["d_model"], dtype=torch.bfloat16, device=dev)
    lay0 = layers_dev[0]
    ws_bytes = max(wl.workspace_bytes(wl.OP_QKV, [lay0["q"], lay0["k"], lay0["v"]], T),
                   wl.workspace_bytes(wl.OP_LINEAR, [lay0["o"]], T),
                   wl.workspace_bytes(wl.OP_MLP, [lay0["gate"], lay0["up"], lay0["down"]], T))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)

    def mlp(l: int):
        lay, a = layers_dev[l], acts_dev[l]
        wl.wl_mlp_fused(lay["gate"], lay["up"], lay["down"], a["x_mlp"], y=y_mlp, ws=ws)

    def step(l: int):
        lay, a = layers_dev[l], acts_dev[l]
        wl.wl_qkv_fused(lay["q"], lay["k"], lay["v"], a["x_attn"], y=y_qkv, ws=ws)
        wl.wl_linear(lay["o"], a["x_o"], y=y_o, ws=ws)
        mlp(l)

    # Parity spot check of layer 0 against the oracle (eager, outside the timed region).
    step(0)
    torch.cuda.synchronize()
    from oracle import oracle as oracle_mod
    orc = oracle_mod.default()
    h0, a0 = host_layer0, host_acts0
    parity = {}
    for name, y_gpu, (y_ref, bound) in (
            ("qkv", y_qkv, orc.qkv(h0["q"], h0["k"], h0["v"], a0["x_attn"])),
            ("o", y_o, orc.linear(h0["o"], a0["x_o"])),
            ("mlp", y_mlp, orc.mlp(h0["gate"], h0["up"], h0["down"], a0["x_mlp"])[:2])):
        yg = y_gpu.float().cpu().double().numpy()
        parity[name] = float(np.linalg.norm(yg - y_ref) / np.linalg.norm(y_ref))

    # At one token a layer is ~10 us of GPU work, less than the host cost of its
    # launches, so steps are replayed from HIP graphs: one graph holding all L
    # layer steps, and one graph per single layer step so that exactly K steps
    # run. The fused MLP of every layer is captured alone as well, for the
    # per-operation timing of the roofline record.
    for l in range(L):
        step(l)
    torch.cuda.synchronize()
    g_all, g_one, g_mlp = torch.cuda.CUDAGraph(), [], torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_all):
        for l in range(L):
            step(l)
    for l in range(L):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(l)
        g_one.append(g)
    with torch.cuda.graph(g_mlp):
        for l in range(L):
            mlp(l)

    def run_steps(n: int):
        for _ in range(n // L):
            g_all.replay()
        for l in range(n % L):
            g_one[l].replay()

    run_steps(args.warmup)
    torch.cuda.synchronize()

    K = args.steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall = time.perf_counter()
    start.record()
    run_steps(K)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall
    ms_total = start.elapsed_time(stop)
    ms_per_step = ms_total / K

    # Dominant operation: the fused MLP, all L layers per replay, timed with HIP
    # events on the launch stream.
    n_mlp = max(1, K // L)
    m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g_mlp.replay()
    m0.record()
    for _ in range(n_mlp):
        g_mlp.replay()
    m1.record()
    torch.cuda.synchronize()
    mlp_ms = m0.elapsed_time(m1) / (n_mlp * L)

    # Algorithmic bytes: every theta tensor once, plus the call's x and y.
    lay0 = host_layer0
    d = dims["d_model"]
    mlp_bytes = sum(theta_bytes(lay0[f]) for f in ("gate", "up", "down")) + 2 * T * d + 2 * T * d
    layer_bytes = (sum(theta_bytes(lay0[f]) for f in inputs.FAMILIES)
                   + 2 * T * (d + width_qkv) + 2 * T * (dims["q"] + d) + 2 * T * (d + d))
    mlp_gbs = mlp_bytes / (mlp_ms * 1e-3) / 1e9
    layer_gbs = layer_bytes / (ms_per_step * 1e-3) / 1e9

    cpu = None
    if args.cpu_seconds > 0:
        reps, t0 = 0, time.perf_counter()
        while True:
            orc.qkv(h0["q"], h0["k"], h0["v"], a0["x_attn"])
            orc.linear(h0["o"], a0["x_o"])
            orc.mlp(h0["gate"], h0["up"], h0["down"], a0["x_mlp"])
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds and reps >= 2:
                break
        cpu = {"value": reps * T / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps} passes of layer 0 (QKV + O + MLP, T=1, r={r}) in {el:.1f} s, "
                         "single-threaded fp64 C oracle"}

    out = {
        "metric": METRIC,
        "value": K * T / (ms_total * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gemma3-1b-shaped layer decode (QKV fused + O + MLP fused)",
                   "T": T, "rank": r, "layers_cycled": L, "G": L, "d_model": d, "q": dims["q"],
                   "kv": dims["kv"], "d_ff": dims["ff"], "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": mlp_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": mlp_gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "wl_mlp_fused (T=1), graph of all layers", "bytes_per_launch": mlp_bytes,
                     "us_per_launch": mlp_ms * 1e3},
        "layer_hbm_gbs": layer_gbs,
        "layer_bytes": layer_bytes,
        "wall_s_timed": wall,
        "parity_rel_l2": parity,
        "cpu_baseline": cpu,
        "setup_s": t_gen,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
