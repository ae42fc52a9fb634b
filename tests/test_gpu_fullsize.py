"""Parity at the full sizes the benchmark times, on sampled outputs.

Each case runs the library call at the workload's full shape (the same calls,
shapes and regime choice as bench.py) and compares a sample of token rows with
the oracle, which computes each token row independently of the others: the
first and last tokens and a few seeded ones. The MLP rows include the whole
chain (gate/up, GELU-tanh, bf16 h, down) for the sampled tokens. W_eff is
compared on sampled rows of the matrix.
"""
from __future__ import annotations

import os

import numpy as np
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


def sample_tokens(T: int, n_extra: int, seed: int) -> list:
    g = torch.Generator().manual_seed(seed)
    extra = torch.randint(0, T, (n_extra,), generator=g).tolist()
    return sorted(set([0, T - 1] + extra))


def run_layer(wl, orc, dims, r, T, seed, n_extra, w0_std=0.02, regime=0):
    g = torch.Generator().manual_seed(seed)
    lay = inputs.layer(g, dims, r, w0_std=w0_std)
    acts = inputs.layer_inputs(g, dims, T)
    dl = {f: wl.theta_to(lay[f], DEV) for f in lay}
    prev = wl.set_regime(regime)
    try:
        y_qkv = wl.wl_qkv_fused(dl["q"], dl["k"], dl["v"], acts["x_attn"].to(DEV))
        y_o = wl.wl_linear(dl["o"], acts["x_o"].to(DEV))
        y_mlp = wl.wl_mlp_fused(dl["gate"], dl["up"], dl["down"], acts["x_mlp"].to(DEV))
        torch.cuda.synchronize()
    finally:
        wl.set_regime(prev)
    rows = sample_tokens(T, n_extra, seed + 1)
    sel = torch.tensor(rows)
    what = f"{dims['d_model']}-layer T={T} r={r} tokens {rows}"
    y_ref, b = orc.qkv(lay["q"], lay["k"], lay["v"], acts["x_attn"][sel])
    check(y_qkv[sel.to(DEV)], y_ref, b, "qkv " + what)
    y_ref, b = orc.linear(lay["o"], acts["x_o"][sel])
    check(y_o[sel.to(DEV)], y_ref, b, "o " + what)
    y_ref, b, _ = orc.mlp(lay["gate"], lay["up"], lay["down"], acts["x_mlp"][sel])
    check(y_mlp[sel.to(DEV)], y_ref, b, "mlp " + what)


@pytest.mark.timeout(300)
def test_prefill_layer_t2048(wl, orc):
    run_layer(wl, orc, inputs.GEMMA3_1B, 32, 2048, 0, 6)


@pytest.mark.parametrize("r", [4, 16, 32])
def test_batched_decode_layer_t32(wl, orc, r):
    run_layer(wl, orc, inputs.GEMMA3_1B, r, 32, 0, 30)


@pytest.mark.parametrize("r", [4, 32])
def test_decode_layer_t1(wl, orc, r):
    run_layer(wl, orc, inputs.GEMMA3_1B, r, 1, 0, 0)


@pytest.mark.timeout(600)
def test_large_layer_t1(wl, orc):
    run_layer(wl, orc, inputs.LARGE_5376, 32, 1, 1, 0, w0_std=0.01)


@pytest.mark.timeout(600)
def test_large_layer_t512(wl, orc):
    run_layer(wl, orc, inputs.LARGE_5376, 32, 512, 1, 2, w0_std=0.01)


def test_shared_w0_layers_t32(wl, orc):
    # G = 1: two layers alias one W0 per family; each layer keeps its own s, U, V.
    g = torch.Generator().manual_seed(7)
    dims = inputs.GEMMA3_1B
    lays = inputs.layers(g, dims, 32, 2, 1)
    assert lays[0]["gate"]["W0"] is lays[1]["gate"]["W0"]
    x = inputs.activations(g, 32, dims["d_model"])
    w0 = {f: lays[0][f]["W0"].to(DEV) for f in inputs.FAMILIES}
    for lay in lays:
        dl = {f: dict(wl.theta_to(lay[f], DEV), W0=w0[f]) for f in inputs.FAMILIES}
        y = wl.wl_mlp_fused(dl["gate"], dl["up"], dl["down"], x.to(DEV))
        rows = sample_tokens(32, 3, 8)
        sel = torch.tensor(rows)
        y_ref, b, _ = orc.mlp(lay["gate"], lay["up"], lay["down"], x[sel])
        check(y[sel.to(DEV)], y_ref, b, "shared-W0 mlp")


def test_weff_full_gate_shape(wl, orc):
    g = torch.Generator().manual_seed(11)
    th = inputs.theta(g, 1152, 6912, 32)
    w = wl.wl_materialize_weff(wl.theta_to(th, DEV))
    rows = sample_tokens(6912, 6, 12)
    sub = dict(th, W0=th["W0"][rows], s=th["s"][rows], U=th["U"][rows], d_out=len(rows))
    w_ref, b = orc.weff(sub)
    check(w[torch.tensor(rows, device=DEV)], w_ref, b, f"W_eff rows {rows}")
    assert np.isfinite(w.float().cpu().numpy()).all()
