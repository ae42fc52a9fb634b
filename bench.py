#!/usr/bin/env python3
"""Benchmark of the fused reconstruct-and-project linear on one MI355X.

    y = s (.) (W0 x) + U (V^T x)      bf16 W0, U, V, x; fp32 s; fp32 accumulate; bf16 y

Workloads (``--workload``; the default is the one the headline metric is quoted on):

  layer-decode    one Gemma-3-1B-shaped decoder layer at T = 1 token, rank r
                  (default 32): fused Q/K/V 1152 -> 1024 + 256 + 256, O 1024 ->
                  1152, fused MLP gate/up 1152 -> 6912, GELU-tanh, down 6912 ->
                  1152. A step is one layer (wl_qkv_fused, wl_linear,
                  wl_mlp_fused); steps cycle over 26 resident layers with their
                  own W0, so the 1.4 GB weight set streams from HBM rather than
                  from the 256 MB last-level cache. Tokens/s are per layer.
  single          one 1152 -> 1152 projection, r = 4, T = 1; steps cycle over 400
                  resident copies (about 1.07 GB).
  batched-decode  the same layer shapes, 26 layers, T = 32 tokens (32 concurrent
                  streams), r (default 32); a step is all 26 layers. --shared-w0
                  gives every layer the same W0 (G = 1), the default is an own W0
                  per layer (G = 26).
  prefill         the same layer shapes at T = 2048 tokens, r = 32; a step is one
                  layer, cycling over 26 layers. Also times wl_materialize_weff for
                  the seven projections of a layer.
  large           a hidden-5376 layer: Q/K/V 5376 -> 8192 + 2048 + 2048, O 8192 ->
                  5376, MLP 5376 -> 21504 -> 5376, r = 32, T = --tokens (1 or
                  512). W0 ~ N(0, 0.01), seed 1. A step is one layer.
  copy            a plain 512 MiB device copy, the reference that scales the
                  FETCH_SIZE / WRITE_SIZE hardware counters to bytes.

For hardware-counter passes, --dominant-only runs just the dominant call, and
--traffic-from turns the passes' counter files into the per-call HBM traffic
that the roofline record reports (profiles/traffic_*.txt, tied to a digest of
the kernel sources; a record whose kernels changed since reports null).

Inputs are seeded synthetic draws (linear_02_amd.inputs) with W0 ~ N(0, 0.02)
(0.01 for large), s ~ 1 + N(0, 0.01), U, V ~ N(0, 0.01), x ~ N(0, 1), already
resident in device memory when timing starts. Steps are replayed from HIP
graphs, since at decode sizes a call is shorter than the host cost of its
launches. The roofline record covers the dominant library call (the fused MLP):
its algorithmic bytes (decode) or flops (prefill, large at T = 512) over its
average duration, timed with HIP events on the stream the library launches on.
The oracle (plain fp64 C) is timed on a bounded sample of the same work, on
the host's OpenMP threads and on one thread. The default workload's line also
carries records of the decode layer at r = 4, the MLP at T = 2048 (its MFMA
roofline) and batched decode over 26 layers that share one W0 (G = 1). A timed
region is one launch of a library step (wl_step_create: one HIP graph the library
records) holding exactly the timed steps. One JSON line is printed.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
if REPO not in sys.path:
    sys.path.insert(0, REPO)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 matrix cores
MFMA_F32_PEAK_TFS = 157.3      # MI355X dense fp32 matrix cores
METRIC = "tokens/s + achieved HBM GB/s (T=1) / MFMA TFLOP/s (T=2048) per rank"
WORKLOADS = ("layer-decode", "single", "batched-decode", "prefill", "large", "copy")
DEFAULT_STEPS = {"layer-decode": 520, "single": 800, "batched-decode": 20, "prefill": 52, "large": 20}


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--workload", choices=WORKLOADS, default="layer-decode")
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--rank", type=int, default=None, help="low-rank r (default per workload)")
    p.add_argument("--tokens", type=int, default=None, help="T for the large workload (1 or 512)")
    p.add_argument("--shared-w0", action="store_true", help="batched-decode: one W0 for all layers (G=1)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle sample budget (0 skips it)")
    p.add_argument("--no-records", action="store_true",
                   help="layer-decode: skip the r=4 decode, T=2048 MLP and shared-W0 batched-decode records")
    p.add_argument("--dominant-only", action="store_true",
                   help="run only the dominant call (for hardware-counter passes) and print the call count")
    p.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                   help="write the dominant call's HBM traffic from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE "
                        "counter files (of a --dominant-only run and of --workload copy) and exit")
    p.add_argument("--traffic-calls", type=int, default=0, help="dominant calls in the counted run")
    p.add_argument("--dtype", choices=("bf16", "f32"), default="bf16",
                   help="element type of W0, U, V, x, y (f32: the fp32 variant of every operation)")
    return p.parse_args()


# -- algorithmic work (counted once per call; what the method must move or compute) ----------

def elem_bytes(th: dict) -> int:
    """Bytes per element of a theta's W0, U, V (and of its call's x, y)."""
    return th["W0"].element_size()


def theta_bytes(th: dict) -> int:
    """W0 + s + U + V bytes of one theta."""
    d_in, d_out, r, e = th["d_in"], th["d_out"], th["r"], elem_bytes(th)
    return e * d_out * d_in + (4 * d_out if th.get("s") is not None else 0) + e * r * (d_out + d_in)


def theta_flops(th: dict, T: int) -> int:
    """Multiply-adds of W0 x, V^T x and U vtx (2 flops each) plus the s scaling."""
    d_in, d_out, r = th["d_in"], th["d_out"], th["r"]
    return 2 * T * d_out * d_in + 2 * T * r * (d_in + d_out) + 2 * T * d_out


def call_bytes(thetas, T: int, d_x: int, d_y: int) -> int:
    e = elem_bytes(thetas[0])
    return sum(theta_bytes(t) for t in thetas) + e * T * d_x + e * T * d_y


def layer_work(lay: dict, dims: dict, T: int):
    """(bytes, flops) of one layer: Q/K/V call, O call, MLP call."""
    d, width = dims["d_model"], dims["q"] + 2 * dims["kv"]
    b = (call_bytes([lay[f] for f in "qkv"], T, d, width) + call_bytes([lay["o"]], T, dims["q"], d)
         + call_bytes([lay[f] for f in ("gate", "up", "down")], T, d, d))
    fl = sum(theta_flops(lay[f], T) for f in ("q", "k", "v", "o", "gate", "up", "down"))
    return b, fl


def mlp_work(lay: dict, dims: dict, T: int):
    d = dims["d_model"]
    b = call_bytes([lay[f] for f in ("gate", "up", "down")], T, d, d)
    fl = sum(theta_flops(lay[f], T) for f in ("gate", "up", "down"))
    return b, fl


# Sources of the kernels that the dominant call (the MLP) runs at each token
# count, which the traffic records measure (the shared device headers always
# count; the host dispatcher does not, so host-only changes such as a new entry
# point leave the records valid): the one-launch MLP (at most 2 tokens), the
# decode GEMV with its V^T x launch, the skinny path, the matrix-core GEMM with
# its V^T x launch.
_COMMON_SOURCES = ("wl_kernels.h", "wl_device.h")
_MLP_ONE_LAUNCH_MAX_TOK = 2


def _regime_sources(tokens: int, dtype: str = "bf16") -> tuple:
    if dtype == "f32":
        return ("k_f32.hip",)
    if tokens <= _MLP_ONE_LAUNCH_MAX_TOK:
        return ("k_mlp.hip", "wl_vtx_slice.h", "wl_handoff.h")
    if tokens <= 8:
        return ("k_gemv.hip", "k_vtx.hip", "wl_vtx_slice.h", "wl_handoff.h")
    if tokens <= 64:
        return ("k_skinny.hip",)
    return ("k_gemm.hip", "k_vtxmm.hip", "wl_vtxmm.h")


def source_digest(tokens: int, dtype: str = "bf16") -> str:
    """Digest of the sources of the kernels that run at this token count, to tell
    whether stored counter data still applies."""
    h = hashlib.sha256()
    for name in sorted(_COMMON_SOURCES + _regime_sources(tokens, dtype)):
        with open(os.path.join(REPO, "linear_02_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_key(args, workload: str) -> str:
    """Name of a workload's traffic record: one W0 shared by all layers (--shared-w0)
    moves other bytes than one W0 per layer, and the fp32 variant other bytes than
    bf16, so each has a record of its own."""
    key = workload + "-G1" if getattr(args, "shared_w0", False) else workload
    return key + "-f32" if getattr(args, "dtype", "bf16") == "f32" else key


def stored_traffic(workload: str, rank: int, tokens: int):
    """HBM bytes per call of the dominant operation from the committed counter summary
    (rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE passes), or None when there is none or
    the kernels changed since it was taken."""
    path = os.path.join(REPO, "profiles", f"traffic_{workload}_r{rank}_T{tokens}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("sources") != source_digest(tokens, "f32" if workload.endswith("-f32") else "bf16"):
        return None
    try:
        return float(kv["bytes_per_call"])
    except (KeyError, ValueError):
        return None


# -- timing -------------------------------------------------------------------------------

class StepGraph:
    """One HIP graph holding exactly k steps, step i running fns[i % len(fns)], so
    that a timed region is one replay whatever k is (no host gaps between steps
    and none that depend on k)."""

    def __init__(self, torch, fns, k: int):
        for fn in fns:      # eager pass: allocations and workspace before capture
            fn()
        torch.cuda.synchronize()
        self.k = k
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for i in range(k):
                fns[i % len(fns)]()

    def replay(self):
        self.graph.replay()


def time_calls(torch, fns, calls: int) -> float:
    """Average ms per call over `calls` calls (cycling over fns) in one graph,
    replayed once to warm up and once timed."""
    g = StepGraph(torch, fns, calls)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / calls


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_sample(orc, budget_s: float, fn, units_per_call: float, unit: str, what: str):
    """Time the oracle on the host's cores (its OpenMP threads: OMP_NUM_THREADS
    when set, else every core the process may run on) and on one thread, each
    for half the budget (at least one call each)."""
    if budget_s <= 0:
        return None

    def rate(seconds):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return reps, el

    threads = orc.threads()
    reps, el = rate(budget_s / 2)
    orc.threads(1)
    try:
        reps1, el1 = rate(budget_s / 2)
    finally:
        orc.threads(threads)
    return {"value": reps * units_per_call / el, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{reps} x {what} in {el:.1f} s, fp64 C oracle on {threads} OpenMP threads",
            "affine_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "single_thread": {"value": reps1 * units_per_call / el1, "unit": unit, "cores": 1,
                              "sample": f"{reps1} x {what} in {el1:.1f} s on one thread"}}


def rel_l2(np, y_gpu, y_ref) -> float:
    yg = y_gpu.float().cpu().double().numpy()
    return float(np.linalg.norm(yg - y_ref) / np.linalg.norm(y_ref))


# -- workloads ----------------------------------------------------------------------------

def build_layers(args, torch, wl, inputs, *, dims, r, n_layers, G, w0_std, seed):
    """Seeded synthetic layers on the host and on the device (W0 blocks shared
    between layers stay shared on the device)."""
    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(seed)
    dt = torch.float32 if args.dtype == "f32" else torch.bfloat16
    host_layers = inputs.layers(gen, dims, r, n_layers, G, w0_std=w0_std, dtype=dt)
    layers = [{f: wl.theta_to(lay[f], dev) for f in inputs.FAMILIES} for lay in host_layers]
    if G < n_layers:
        band = -(-n_layers // G)
        for l in range(n_layers):
            for f in inputs.FAMILIES:
                layers[l][f]["W0"] = layers[(l // band) * band][f]["W0"]
    return gen, host_layers, layers


class LayerCalls:
    """The three library calls of a decoder layer at T tokens, on preallocated
    outputs and one workspace."""

    def __init__(self, torch, wl, inputs, gen, layers, dims, T, dt):
        dev = torch.device("cuda:0")
        self.wl, self.layers = wl, layers
        self.acts = inputs.layer_inputs(gen, dims, T, dtype=dt)
        self.xa = {k: v.to(dev) for k, v in self.acts.items()}
        d, width = dims["d_model"], dims["q"] + 2 * dims["kv"]
        self.y_qkv = torch.empty(T, width, dtype=dt, device=dev)
        self.y_o = torch.empty(T, d, dtype=dt, device=dev)
        self.y_mlp = torch.empty(T, d, dtype=dt, device=dev)
        l0 = layers[0]
        ws_bytes = max(wl.workspace_bytes(wl.OP_QKV, [l0["q"], l0["k"], l0["v"]], T),
                       wl.workspace_bytes(wl.OP_LINEAR, [l0["o"]], T),
                       wl.workspace_bytes(wl.OP_MLP, [l0["gate"], l0["up"], l0["down"]], T))
        self.ws = wl.new_workspace(ws_bytes, dev)

    def qkv(self, l):
        lay = self.layers[l]
        self.wl.wl_qkv_fused(lay["q"], lay["k"], lay["v"], self.xa["x_attn"], y=self.y_qkv, ws=self.ws)

    def o(self, l):
        self.wl.wl_linear(self.layers[l]["o"], self.xa["x_o"], y=self.y_o, ws=self.ws)

    def mlp(self, l):
        lay = self.layers[l]
        self.wl.wl_mlp_fused(lay["gate"], lay["up"], lay["down"], self.xa["x_mlp"], y=self.y_mlp, ws=self.ws)

    def step(self, l):
        self.qkv(l)
        self.o(l)
        self.mlp(l)

    # the same calls as (op, thetas, x, y) tuples for a library step
    def call_mlp(self, l):
        lay = self.layers[l]
        return (self.wl.OP_MLP, [lay["gate"], lay["up"], lay["down"]], self.xa["x_mlp"], self.y_mlp)

    def calls(self, l):
        lay = self.layers[l]
        return [(self.wl.OP_QKV, [lay["q"], lay["k"], lay["v"]], self.xa["x_attn"], self.y_qkv),
                (self.wl.OP_LINEAR, [lay["o"]], self.xa["x_o"], self.y_o),
                self.call_mlp(l)]


def time_library_steps(torch, wl, step_calls, steps: int, warmup: int, ws):
    """(ms, wall s) of exactly `steps` steps made into one library step (one HIP
    graph recorded by wl_step_create and launched by wl_step_launch), after
    `warmup` steps in another; step_calls(i) lists step i's calls."""
    timed = wl.Step([c for i in range(steps) for c in step_calls(i)], ws=ws)
    if warmup > 0:
        warm = wl.Step([c for i in range(warmup) for c in step_calls(i)], ws=ws)
        warm.launch()
        torch.cuda.synchronize()
        warm.close()
    timed.launch()   # first launch of the graph: upload, outside the timed region
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall = time.perf_counter()
    e0.record()
    timed.launch()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall
    timed.close()
    return e0.elapsed_time(e1), wall


def hbm_roof(bytes_per_launch, ms, traffic, kernel):
    achieved = bytes_per_launch / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": kernel,
            "bytes_per_launch": bytes_per_launch, "us_per_launch": ms * 1e3}


def mfma_roof(flops_per_launch, ms, traffic, kernel, peak):
    achieved = flops_per_launch / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak, "traffic": traffic, "kernel": kernel,
            "flops_per_launch": flops_per_launch, "us_per_launch": ms * 1e3}


def mlp_kernel_name(T: int) -> str:
    if T <= 2:
        return "wl_mlp_fused: one launch (gate/up, GELU-tanh and down together)"
    return "wl_mlp_fused (all of its kernels, back to back)"


def run_layers(args, torch, np, wl, inputs, orc, *, dims, r, T, n_layers, G, w0_std, seed, workload,
               bound):
    """Decoder-layer workloads: steps of one layer (or of all layers for batched decode)."""
    t_gen = time.perf_counter()
    dt = torch.float32 if args.dtype == "f32" else torch.bfloat16
    gen, host_layers, layers = build_layers(args, torch, wl, inputs, dims=dims, r=r, n_layers=n_layers, G=G,
                                            w0_std=w0_std, seed=seed)
    calls = LayerCalls(torch, wl, inputs, gen, layers, dims, T, dt)
    acts = calls.acts
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    if args.dominant_only:
        n = args.steps if args.steps is not None else n_layers
        for i in range(n):
            calls.mlp(i % n_layers)
        torch.cuda.synchronize()
        print(json.dumps({"dominant_calls": n, "call": "wl_mlp_fused", "workload": workload}))
        return None

    # Parity spot check of layer 0 against the oracle (eager, outside the timed region).
    calls.step(0)
    torch.cuda.synchronize()
    h0 = host_layers[0]
    parity = {}
    if T <= 64 or workload == "prefill":
        # At prefill sizes the oracle takes a slice of the tokens: the first 16.
        n_chk = min(T, 16)
        sl = slice(0, n_chk)
        parity["qkv"] = rel_l2(np, calls.y_qkv[sl], orc.qkv(h0["q"], h0["k"], h0["v"], acts["x_attn"][sl])[0])
        parity["o"] = rel_l2(np, calls.y_o[sl], orc.linear(h0["o"], acts["x_o"][sl])[0])
        parity["mlp"] = rel_l2(np, calls.y_mlp[sl],
                               orc.mlp(h0["gate"], h0["up"], h0["down"], acts["x_mlp"][sl])[0])
        parity["tokens_checked"] = n_chk

    if workload == "batched-decode":
        def step_calls(i):
            return [c for l in range(n_layers) for c in calls.calls(l)]
        unit_layers = n_layers
    else:
        def step_calls(i):
            return calls.calls(i % n_layers)
        unit_layers = 1
    mlp_fns = [lambda l=l: calls.mlp(l) for l in range(n_layers)]

    K = args.steps if args.steps is not None else DEFAULT_STEPS[workload]
    W = args.warmup if args.warmup is not None else max(1, K // 10)
    ms_total, wall = time_library_steps(torch, wl, step_calls, K, W, calls.ws)
    ms_per_step = ms_total / K
    mlp_ms = time_calls(torch, mlp_fns, max(10 * n_layers, 260))

    lay_b, lay_f = layer_work(h0, dims, T)
    mlp_b, mlp_f = mlp_work(h0, dims, T)
    step_b, step_f = lay_b * unit_layers, lay_f * unit_layers
    traffic = stored_traffic(traffic_key(args, workload), r, T)
    if bound == "hbm":
        roof = hbm_roof(mlp_b, mlp_ms, traffic, mlp_kernel_name(T))
    else:
        peak = MFMA_F32_PEAK_TFS if args.dtype == "f32" else MFMA_BF16_PEAK_TFS
        roof = mfma_roof(mlp_f, mlp_ms, traffic, mlp_kernel_name(T), peak)

    # Oracle sample: whole layers at decode sizes, a few tokens of a layer otherwise.
    n_tok = T if T <= 32 else (8 if T <= 512 else 4)
    sl = slice(0, n_tok)

    def oracle_layer():
        orc.qkv(h0["q"], h0["k"], h0["v"], acts["x_attn"][sl])
        orc.linear(h0["o"], acts["x_o"][sl])
        orc.mlp(h0["gate"], h0["up"], h0["down"], acts["x_mlp"][sl])

    cpu = oracle_sample(orc, args.cpu_seconds, oracle_layer, n_tok, "tokens/s",
                        f"one layer (QKV + O + MLP) at {n_tok} token(s), r={r}")

    extra = {}
    if workload == "prefill":
        extra.update(materialize_and_dense(torch, wl, layers, calls.xa, dims, T, calls.ws))
    if workload == "layer-decode" and args.dtype == "bf16" and not args.no_records:
        records = {}
        # records use a fixed step count: they are not the headline, and a few
        # steps right after their layers are made time noisily
        records["decode_r4"] = record_decode(args, torch, wl, inputs, dims, n_layers, 4, 260, 26)
        records["prefill_mlp_T2048_r32"] = record_prefill_mlp(args, torch, wl, inputs, gen, layers, h0, dims)
        records["batched_decode_G1_T32_r32"] = record_batched_g1(args, torch, wl, inputs, dims)
        extra["records"] = records

    out = {
        "value": K * T / (ms_total * 1e-3),
        "unit": "tokens/s",
        "steps": K, "warmup": W, "ms_per_step": ms_per_step,
        "config": {"workload": workload_name(workload, dims, r, T, n_layers, G)
                   + (", fp32 weights and activations" if args.dtype == "f32" else ""),
                   "T": T, "rank": r, "layers": n_layers, "G": G, "d_model": dims["d_model"], "q": dims["q"],
                   "kv": dims["kv"], "d_ff": dims["ff"], "parallelism": "single-gpu"},
        "roofline": roof,
        "step_hbm_gbs": step_b / (ms_per_step * 1e-3) / 1e9,
        "step_tflops": step_f / (ms_per_step * 1e-3) / 1e12,
        "step_bytes": step_b, "step_flops": step_f,
        "wall_s_timed": wall,
        "parity_rel_l2": parity,
        "cpu_baseline": cpu,
        "setup_s": t_gen,
    }
    out.update(extra)
    return out


def record_decode(args, torch, wl, inputs, dims, n_layers, r, K, W):
    """The decode layer at another rank: tokens/s per layer over the same step
    count, and the MLP call's HBM roofline."""
    dt = torch.bfloat16
    gen, host_layers, layers = build_layers(args, torch, wl, inputs, dims=dims, r=r, n_layers=n_layers,
                                            G=n_layers, w0_std=0.02, seed=0)
    calls = LayerCalls(torch, wl, inputs, gen, layers, dims, 1, dt)
    ms_total, _ = time_library_steps(torch, wl, lambda i: calls.calls(i % n_layers), K, W, calls.ws)
    mlp_ms = time_calls(torch, [lambda l=l: calls.mlp(l) for l in range(n_layers)], max(10 * n_layers, 260))
    mlp_b, _ = mlp_work(host_layers[0], dims, 1)
    lay_b, _ = layer_work(host_layers[0], dims, 1)
    rec = {"workload": f"gemma3-1b-shaped layer decode, T=1, r={r}, per layer, 26 resident layers",
           "tokens_per_s": K / (ms_total * 1e-3), "us_per_layer": ms_total * 1e3 / K, "steps": K,
           "layer_hbm_gbs": lay_b / (ms_total * 1e-3 / K) / 1e9,
           "roofline": hbm_roof(mlp_b, mlp_ms, stored_traffic("layer-decode", r, 1), mlp_kernel_name(1))}
    del layers, calls
    torch.cuda.empty_cache()
    return rec


def record_prefill_mlp(args, torch, wl, inputs, gen, layers, h0, dims):
    """The MLP call at T = 2048 (r = 32, the headline's 26 layers): its MFMA
    roofline, timed over 26 calls, one per layer."""
    T = 2048
    calls = LayerCalls(torch, wl, inputs, gen, layers, dims, T, torch.bfloat16)
    n = len(layers)
    mlp_ms = time_calls(torch, [lambda l=l: calls.mlp(l) for l in range(n)], 2 * n)
    lay_ms = time_calls(torch, [lambda l=l: calls.step(l) for l in range(n)], n)
    mlp_b, mlp_f = mlp_work(h0, dims, T)
    lay_b, lay_f = layer_work(h0, dims, T)
    rec = {"workload": "gemma3-1b-shaped MLP prefill, T=2048, r=32 (gate/up 1152 -> 6912, down 6912 -> 1152)",
           "tokens_per_s_mlp": T / (mlp_ms * 1e-3),
           "layer_us": lay_ms * 1e3, "layer_tflops": lay_f / (lay_ms * 1e-3) / 1e12,
           "roofline": mfma_roof(mlp_f, mlp_ms, stored_traffic("prefill", 32, T), mlp_kernel_name(T),
                                 MFMA_BF16_PEAK_TFS)}
    del calls
    torch.cuda.empty_cache()
    return rec


def record_batched_g1(args, torch, wl, inputs, dims):
    """Batched decode (T = 32) over 26 layers that share one W0 per family (G = 1):
    tokens/s of a 26-layer step, and its algorithmic bytes (every call's operands
    counted), unique bytes (the one W0 set once, every layer's s, U, V, every
    call's x and y) and the counter bytes of the MLP call from its traffic record.
    The step is timed in the given layer order and, with every layer's calls
    given outputs of their own (so that they are independent), regrouped so the
    26 calls sharing a W0 run back to back (WL_STEP_GROUP_SHARED_W0)."""
    T, n_layers, r = 32, 26, 32
    gen, host_layers, layers = build_layers(args, torch, wl, inputs, dims=dims, r=r, n_layers=n_layers, G=1,
                                            w0_std=0.02, seed=0)
    calls = LayerCalls(torch, wl, inputs, gen, layers, dims, T, torch.bfloat16)
    all_layers = [c for l in range(n_layers) for c in calls.calls(l)]
    ms, _ = time_library_steps(torch, wl, lambda i: all_layers, 4, 1, calls.ws)
    ms /= 4
    # independent calls: outputs of their own per layer
    own = []
    for l in range(n_layers):
        for op, ths, x, y in calls.calls(l):
            own.append((op, ths, x, torch.empty_like(y)))
    grouped = wl.Step(own * 1, ws=calls.ws, group_shared_w0=True)
    grouped.launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(4):
        grouped.launch()
    e1.record()
    torch.cuda.synchronize()
    ms_grouped = e0.elapsed_time(e1) / 4
    grouped.close()
    mlp_ms = time_calls(torch, [lambda l=l: calls.mlp(l) for l in range(n_layers)], 2 * n_layers)
    h0 = host_layers[0]
    lay_b, _ = layer_work(h0, dims, T)
    w0_once = sum(h0[f]["W0"].numel() * h0[f]["W0"].element_size() for f in inputs.FAMILIES)
    unique = n_layers * lay_b - (n_layers - 1) * w0_once
    mlp_b, _ = mlp_work(h0, dims, T)
    mlp_w0 = sum(h0[f]["W0"].numel() * h0[f]["W0"].element_size() for f in ("gate", "up", "down"))
    rec = {"workload": "gemma3-1b-shaped 26 layers sharing one W0 per family (G=1), batched decode T=32, r=32",
           "tokens_per_s": T / (ms * 1e-3), "ms_per_26_layer_step": ms,
           "ms_per_26_layer_step_grouped_by_w0": ms_grouped,
           "algorithmic_bytes_per_step": n_layers * lay_b, "unique_bytes_per_step": unique,
           "mlp_call": {"us": mlp_ms * 1e3, "algorithmic_bytes": mlp_b,
                        "unique_bytes_26_calls": n_layers * mlp_b - (n_layers - 1) * mlp_w0,
                        "counter_bytes": stored_traffic("batched-decode-G1", r, T)}}
    del layers, calls, own
    torch.cuda.empty_cache()
    return rec


def materialize_and_dense(torch, wl, layers, xa, dims, T, ws):
    """The precompute-outside path at prefill: W_eff for the seven projections of a
    layer, and the dense products with those W_eff (s = 1, r = 0 through the same
    library), against the fused path."""
    dev = layers[0]["q"]["W0"].device
    lay = layers[0]
    weff = {f: torch.empty_like(lay[f]["W0"]) for f in lay}

    fams = list(lay)

    def materialize():
        wl.wl_materialize_weff_batch([lay[f] for f in fams], [weff[f] for f in fams])

    def materialize_each():
        for f in fams:
            wl.wl_materialize_weff(lay[f], W_eff=weff[f])

    dense = {f: dict(W0=weff[f], s=None, U=None, V=None, d_in=lay[f]["d_in"], d_out=lay[f]["d_out"], r=0)
             for f in lay}
    d, width = dims["d_model"], dims["q"] + 2 * dims["kv"]
    dt = lay["q"]["W0"].dtype
    y_qkv = torch.empty(T, width, dtype=dt, device=dev)
    y_o = torch.empty(T, d, dtype=dt, device=dev)
    y_mlp = torch.empty(T, d, dtype=dt, device=dev)

    def dense_layer():
        wl.wl_qkv_fused(dense["q"], dense["k"], dense["v"], xa["x_attn"], y=y_qkv, ws=ws)
        wl.wl_linear(dense["o"], xa["x_o"], y=y_o, ws=ws)
        wl.wl_mlp_fused(dense["gate"], dense["up"], dense["down"], xa["x_mlp"], y=y_mlp, ws=ws)

    m_ms = time_calls(torch, [materialize], 20)
    m1_ms = time_calls(torch, [materialize_each], 20)
    d_ms = time_calls(torch, [dense_layer], 20)
    e = lay["q"]["W0"].element_size()
    w_bytes = sum(2 * e * lay[f]["d_out"] * lay[f]["d_in"] + 4 * lay[f]["d_out"]
                  + e * lay[f]["r"] * (lay[f]["d_in"] + lay[f]["d_out"]) for f in lay)
    return {"materialize_weff": {"us_per_layer": m_ms * 1e3, "hbm_gbs": w_bytes / (m_ms * 1e-3) / 1e9,
                                 "bytes_per_layer": w_bytes, "call": "wl_materialize_weff_batch (7 projections)",
                                 "us_per_layer_one_call_each": m1_ms * 1e3},
            "dense_on_weff": {"us_per_layer": d_ms * 1e3}}


def workload_name(workload, dims, r, T, n_layers, G):
    if workload == "large":
        return f"hidden-5376 layer (QKV fused + O + MLP fused), T={T}, r={r}, per layer"
    if workload == "batched-decode":
        return f"gemma3-1b-shaped {n_layers} layers, batched decode T={T}, r={r}, G={G}"
    if workload == "prefill":
        return f"gemma3-1b-shaped layer prefill T={T}, r={r}, per layer ({n_layers} resident layers)"
    return (f"gemma3-1b-shaped layer decode (QKV fused + O + MLP fused), T={T}, r={r}, per layer "
            f"({n_layers} resident layers)")


def run_single(args, torch, np, wl, inputs, orc):
    dev = torch.device("cuda:0")
    r, T, d, copies = (args.rank if args.rank is not None else 4), 1, 1152, 400
    gen = torch.Generator().manual_seed(0)
    host = inputs.theta(gen, d, d, r)
    x_host = inputs.activations(gen, T, d)
    # The copies share s, U and V draws and differ in W0 only (fresh draws are slow on
    # the host); every call still reads its own 2.65 MB W0 from HBM.
    ths = []
    for c in range(copies):
        th = wl.theta_to(host, dev)
        if c > 0:
            th["W0"] = torch.randn(d, d, generator=gen).mul_(0.02).to(torch.bfloat16).to(dev)
        ths.append(th)
    x = x_host.to(dev)
    y = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
    ws = wl.new_workspace(wl.workspace_bytes(wl.OP_LINEAR, [ths[0]], T), dev)
    if args.dominant_only:
        n = args.steps if args.steps is not None else copies
        for i in range(n):
            wl.wl_linear(ths[i % copies], x, y=y, ws=ws)
        torch.cuda.synchronize()
        print(json.dumps({"dominant_calls": n, "call": "wl_linear", "workload": "single"}))
        return None
    wl.wl_linear(ths[0], x, y=y, ws=ws)
    torch.cuda.synchronize()
    parity = {"linear": rel_l2(np, y, orc.linear(host, x_host)[0])}
    K = args.steps if args.steps is not None else DEFAULT_STEPS["single"]
    W = args.warmup if args.warmup is not None else max(1, K // 10)
    ms_total, wall = time_library_steps(torch, wl, lambda i: [(wl.OP_LINEAR, [ths[i % copies]], x, y)], K, W, ws)
    ms = ms_total / K
    b = call_bytes([host], T, d, d)
    achieved = b / (ms * 1e-3) / 1e9
    cpu = oracle_sample(orc, args.cpu_seconds, lambda: orc.linear(host, x_host), 1, "tokens/s",
                        f"one 1152->1152 projection at T=1, r={r}")
    return {
        "value": K * T / (ms_total * 1e-3), "unit": "tokens/s", "steps": K, "warmup": W, "ms_per_step": ms,
        "config": {"workload": f"single projection 1152->1152, T=1, r={r}, {copies} resident copies",
                   "T": T, "rank": r, "copies": copies, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": stored_traffic("single", r, T),
                     "kernel": "wl_linear (all of its kernels, back to back)", "bytes_per_launch": b,
                     "us_per_launch": ms * 1e3},
        "wall_s_timed": wall, "parity_rel_l2": parity, "cpu_baseline": cpu,
    }


COPY_BYTES = 512 << 20


def run_copy(args, torch):
    """A plain device copy of known size: the reference for scaling the FETCH_SIZE and
    WRITE_SIZE counters to bytes."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    K = args.steps if args.steps is not None else 20
    for _ in range(K):
        torch.mul(src, 1.0, out=dst)      # one elementwise kernel: reads and writes the buffer once
    torch.cuda.synchronize()
    return {"metric": "device copy for counter calibration", "bytes_read_per_copy": COPY_BYTES,
            "bytes_written_per_copy": COPY_BYTES, "copies": K}


def _counter_rows(path: str, counter: str):
    import csv
    rows = []
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") == counter:
                rows.append((row["Kernel_Name"], float(row["Counter_Value"])))
    return rows


def write_traffic(args) -> int:
    """Per-call HBM bytes of the dominant call from the counter passes, each counter
    scaled by what it reads for the plain copy of known size."""
    fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.traffic_from
    copy_f = [v for n, v in _counter_rows(cfetch_csv, "FETCH_SIZE") if "elementwise" in n or "copy" in n.lower()]
    copy_w = [v for n, v in _counter_rows(cwrite_csv, "WRITE_SIZE") if "elementwise" in n or "copy" in n.lower()]
    # The copy dispatches are the ones that move the full buffer: the largest values.
    kf = COPY_BYTES / (max(copy_f) * 1024.0)
    kw = COPY_BYTES / (max(copy_w) * 1024.0)
    f_kib = sum(v for n, v in _counter_rows(fetch_csv, "FETCH_SIZE") if "wl::" in n)
    w_kib = sum(v for n, v in _counter_rows(write_csv, "WRITE_SIZE") if "wl::" in n)
    calls = args.traffic_calls
    if calls <= 0:
        print("--traffic-calls is required", file=sys.stderr)
        return 2
    per_call = (f_kib * 1024.0 * kf + w_kib * 1024.0 * kw) / calls
    r = args.rank if args.rank is not None else (4 if args.workload == "single" else 32)
    T = {"single": 1, "layer-decode": 1, "batched-decode": 32, "prefill": 2048}.get(
        args.workload, args.tokens if args.tokens is not None else 1)
    path = os.path.join(REPO, "profiles", f"traffic_{traffic_key(args, args.workload)}_r{r}_T{T}.txt")
    def rel(pth):
        return os.path.relpath(os.path.dirname(os.path.abspath(pth)), REPO)
    run = (f"python3 bench.py --workload {args.workload} --rank {r}" + (" --shared-w0" if args.shared_w0 else "")
           + (" --dtype f32" if args.dtype == "f32" else ""))
    with open(path, "w") as f:
        f.write(f"# HBM traffic of the dominant call of bench.py --workload {args.workload} (r={r}, T={T}),\n"
                f"# from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE passes over a --dominant-only run,\n"
                f"# each scaled by the counter's reading for a plain {COPY_BYTES >> 20} MiB device copy.\n"
                f"# Commands (repository root):\n"
                f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d {rel(fetch_csv)} -o p -- {run} --dominant-only --steps {calls}\n"
                f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d {rel(write_csv)} -o p -- {run} --dominant-only --steps {calls}\n"
                f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d {rel(cfetch_csv)} -o p -- python3 bench.py --workload copy --steps 4\n"
                f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d {rel(cwrite_csv)} -o p -- python3 bench.py --workload copy --steps 4\n"
                f"#   {run} --traffic-calls {calls} --traffic-from {' '.join(os.path.relpath(os.path.abspath(c), REPO) for c in args.traffic_from)}\n")
        f.write(f"sources = {source_digest(T, args.dtype)}\n")
        f.write(f"calls = {calls}\n")
        f.write(f"fetch_kib_total = {f_kib:.1f}\nwrite_kib_total = {w_kib:.1f}\n")
        f.write(f"copy_fetch_scale = {kf:.4f}\ncopy_write_scale = {kw:.4f}\n")
        f.write(f"bytes_per_call = {per_call:.0f}\n")
    print(path)
    return 0


def main() -> int:
    args = parse_args()
    if args.traffic_from:
        return write_traffic(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path is single-device; how it would shard is described in DESIGN.md)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from linear_02_amd import build as wl_build
    if not os.path.exists(wl_build.LIBRARY):
        wl_build.build()
    from linear_02_amd import inputs, wl
    from oracle import oracle as oracle_mod

    torch.cuda.set_device(0)
    wk = args.workload
    if wk == "copy":
        print(json.dumps(run_copy(args, torch)))
        return 0
    orc = oracle_mod.default()
    if wk == "single" and args.dtype != "bf16":
        print("--workload single runs bf16 only", file=sys.stderr)
        return 2
    if wk == "single":
        res = run_single(args, torch, np, wl, inputs, orc)
    elif wk == "layer-decode":
        res = run_layers(args, torch, np, wl, inputs, orc, dims=inputs.GEMMA3_1B,
                         r=args.rank if args.rank is not None else 32, T=1, n_layers=26, G=26,
                         w0_std=0.02, seed=0, workload=wk, bound="hbm")
    elif wk == "batched-decode":
        res = run_layers(args, torch, np, wl, inputs, orc, dims=inputs.GEMMA3_1B,
                         r=args.rank if args.rank is not None else 32, T=32, n_layers=26,
                         G=1 if args.shared_w0 else 26, w0_std=0.02, seed=0, workload=wk, bound="hbm")
    elif wk == "prefill":
        res = run_layers(args, torch, np, wl, inputs, orc, dims=inputs.GEMMA3_1B,
                         r=args.rank if args.rank is not None else 32, T=2048, n_layers=26, G=26,
                         w0_std=0.02, seed=0, workload=wk, bound="mfma")
    else:
        T = args.tokens if args.tokens is not None else 1
        res = run_layers(args, torch, np, wl, inputs, orc, dims=inputs.LARGE_5376,
                         r=args.rank if args.rank is not None else 32, T=T, n_layers=1, G=1,
                         w0_std=0.01, seed=1, workload=wk, bound="hbm" if T <= 64 else "mfma")
    if res is None:
        return 0
    out = {"metric": METRIC, "value": res.pop("value"), "unit": res.pop("unit"), "n_gpus": 1,
           "steps": res.pop("steps"), "warmup": res.pop("warmup"), "ms_per_step": res.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.dtype,
           "data": "synthetic"}
    out.update(res)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
