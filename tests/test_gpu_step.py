"""Decode steps: calls recorded once into a HIP graph by the library and launched
with one call (wl_step_create / wl_step_launch).

Checked against the oracle on every launch, with new inputs written between
launches, in every regime (the regime is read when the step is made), and bit
for bit against the same calls made one by one; a call that reads an earlier
call's output; and the shared-W0 regrouping (G = 1: the calls that share a W0
back to back) against the given order, bit for bit.
"""
from __future__ import annotations

import os

import pytest
import torch

from linear_02_amd import inputs
from parity import check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def wl():
    from linear_02_amd import build
    if not os.path.exists(build.LIBRARY):
        build.build()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from linear_02_amd import wl as mod
    return mod


def make_layers(wl, n_layers, G, r, seed):
    g = torch.Generator().manual_seed(seed)
    dims = inputs.GEMMA3_1B
    host = inputs.layers(g, dims, r, n_layers, G)
    dev = [{f: wl.theta_to(lay[f], DEV) for f in inputs.FAMILIES} for lay in host]
    if G < n_layers:   # shared W0 blocks stay shared on the device
        band = -(-n_layers // G)
        for l in range(n_layers):
            for f in inputs.FAMILIES:
                dev[l][f]["W0"] = dev[(l // band) * band][f]["W0"]
    return g, dims, host, dev


def layer_buffers(dims, T, n_layers):
    width = dims["q"] + 2 * dims["kv"]
    bf = torch.bfloat16
    return [dict(x_attn=torch.empty(T, dims["d_model"], dtype=bf, device=DEV),
                 x_o=torch.empty(T, dims["q"], dtype=bf, device=DEV),
                 x_mlp=torch.empty(T, dims["d_model"], dtype=bf, device=DEV),
                 y_qkv=torch.empty(T, width, dtype=bf, device=DEV),
                 y_o=torch.empty(T, dims["d_model"], dtype=bf, device=DEV),
                 y_mlp=torch.empty(T, dims["d_model"], dtype=bf, device=DEV)) for _ in range(n_layers)]


def layer_calls(wl, dev, bufs):
    calls = []
    for lay, b in zip(dev, bufs):
        calls.append((wl.OP_QKV, [lay["q"], lay["k"], lay["v"]], b["x_attn"], b["y_qkv"]))
        calls.append((wl.OP_LINEAR, [lay["o"]], b["x_o"], b["y_o"]))
        calls.append((wl.OP_MLP, [lay["gate"], lay["up"], lay["down"]], b["x_mlp"], b["y_mlp"]))
    return calls


def fill_inputs(g, dims, T, bufs):
    host = []
    for b in bufs:
        acts = inputs.layer_inputs(g, dims, T)
        for k in ("x_attn", "x_o", "x_mlp"):
            b[k].copy_(acts[k].to(DEV))
        host.append(acts)
    return host


@pytest.mark.parametrize("T", [1, 4, 32])
@pytest.mark.parametrize("regime", [0, 1, 2, 3, 4, 5])
def test_step_matches_oracle_across_launches(wl, orc, regime, T):
    n_layers = 2
    g, dims, host, dev = make_layers(wl, n_layers, n_layers, 32, 300 + T)
    bufs = layer_buffers(dims, T, n_layers)
    fill_inputs(g, dims, T, bufs)
    prev = wl.set_regime(regime)
    try:
        step = wl.Step(layer_calls(wl, dev, bufs))
        for launch in range(3):
            acts = fill_inputs(g, dims, T, bufs)
            print(f"step regime {regime} T={T} launch {launch}", flush=True)
            step.launch()
            torch.cuda.synchronize()
            got = [{k: b[k].clone() for k in ("y_qkv", "y_o", "y_mlp")} for b in bufs]
            # the same calls one by one, in the same regime
            for lay, b in zip(dev, bufs):
                wl.wl_qkv_fused(lay["q"], lay["k"], lay["v"], b["x_attn"], y=b["y_qkv"])
                wl.wl_linear(lay["o"], b["x_o"], y=b["y_o"])
                wl.wl_mlp_fused(lay["gate"], lay["up"], lay["down"], b["x_mlp"], y=b["y_mlp"])
            torch.cuda.synchronize()
            for l in range(n_layers):
                for k in ("y_qkv", "y_o", "y_mlp"):
                    assert torch.equal(got[l][k].view(torch.int16), bufs[l][k].view(torch.int16)), \
                        f"layer {l} {k}: step differs from the calls made one by one (launch {launch})"
                h, a = host[l], acts[l]
                what = f"step regime {regime} T={T} launch {launch} layer {l}"
                check(got[l]["y_qkv"], *orc.qkv(h["q"], h["k"], h["v"], a["x_attn"]), "qkv " + what)
                check(got[l]["y_o"], *orc.linear(h["o"], a["x_o"]), "o " + what)
                y_ref, bound, _ = orc.mlp(h["gate"], h["up"], h["down"], a["x_mlp"])
                check(got[l]["y_mlp"], y_ref, bound, "mlp " + what)
        step.close()
    finally:
        wl.set_regime(prev)


@pytest.mark.parametrize("T", [1, 32])
def test_step_call_reads_an_earlier_output(wl, T):
    # O's output is the MLP's input (d_model = 1152 both): the step keeps the order.
    g, dims, host, dev = make_layers(wl, 1, 1, 32, 400 + T)
    bufs = layer_buffers(dims, T, 1)
    fill_inputs(g, dims, T, bufs)
    lay, b = dev[0], bufs[0]
    calls = [(wl.OP_LINEAR, [lay["o"]], b["x_o"], b["y_o"]),
             (wl.OP_MLP, [lay["gate"], lay["up"], lay["down"]], b["y_o"], b["y_mlp"])]
    step = wl.Step(calls)
    for launch in range(2):
        b["x_o"].copy_(inputs.activations(g, T, dims["q"]).to(DEV))
        step.launch()
        torch.cuda.synchronize()
        y = b["y_mlp"].clone()
        y_o = wl.wl_linear(lay["o"], b["x_o"])
        y_ref = wl.wl_mlp_fused(lay["gate"], lay["up"], lay["down"], y_o)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"chain differs at launch {launch}"
    step.close()


@pytest.mark.parametrize("T", [1, 32])
def test_step_grouped_shared_w0_matches_given_order(wl, orc, T):
    # G = 1: four layers alias one W0 per family; independent calls (own inputs
    # and outputs) regrouped so the calls sharing a W0 run back to back.
    n_layers = 4
    g, dims, host, dev = make_layers(wl, n_layers, 1, 32, 500 + T)
    assert dev[0]["gate"]["W0"].data_ptr() == dev[3]["gate"]["W0"].data_ptr()
    bufs = layer_buffers(dims, T, n_layers)
    acts = fill_inputs(g, dims, T, bufs)
    calls = layer_calls(wl, dev, bufs)
    plain = wl.Step(calls)
    grouped = wl.Step(calls, group_shared_w0=True)
    outs = {}
    for name, step in (("given", plain), ("grouped", grouped)):
        for _ in range(2):
            step.launch()
        torch.cuda.synchronize()
        outs[name] = [{k: b[k].clone() for k in ("y_qkv", "y_o", "y_mlp")} for b in bufs]
    for l in range(n_layers):
        for k in ("y_qkv", "y_o", "y_mlp"):
            assert torch.equal(outs["given"][l][k].view(torch.int16), outs["grouped"][l][k].view(torch.int16))
    h, a = host[3], acts[3]
    y_ref, bound, _ = orc.mlp(h["gate"], h["up"], h["down"], a["x_mlp"])
    check(outs["grouped"][3]["y_mlp"], y_ref, bound, f"grouped shared-W0 mlp T={T}")
    plain.close()
    grouped.close()
