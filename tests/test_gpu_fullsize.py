"""Parity at the full sizes the benchmark times.

Each case runs the library call at the workload's full shape (the same calls,
shapes and regime choice as bench.py) and compares it with the oracle (row-
parallel over the host's cores). The T=2048 prefill layer and the large layer
at T=512 compare every element of Q/K/V, O and the MLP (the whole chain:
gate/up, GELU-tanh, bf16 h, down), so every tile of the widest matrix-core
plans (256-row tiles, the input-axis split, the XCD-banded tile order) is
checked; the shorter cases compare the first and last tokens and a few seeded
ones, or every token where that is cheap. W_eff is compared on sampled rows of
the matrix.
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
    """n_extra None compares every token row."""
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
    rows = list(range(T)) if n_extra is None else sample_tokens(T, n_extra, seed + 1)
    sel = torch.tensor(rows)
    what = f"{dims['d_model']}-layer T={T} r={r} " + ("all tokens" if n_extra is None else f"tokens {rows}")
    print(f"oracle for {what}", flush=True)
    y_ref, b = orc.qkv(lay["q"], lay["k"], lay["v"], acts["x_attn"][sel])
    check(y_qkv[sel.to(DEV)], y_ref, b, "qkv " + what)
    y_ref, b = orc.linear(lay["o"], acts["x_o"][sel])
    check(y_o[sel.to(DEV)], y_ref, b, "o " + what)
    y_ref, b, _ = orc.mlp(lay["gate"], lay["up"], lay["down"], acts["x_mlp"][sel])
    check(y_mlp[sel.to(DEV)], y_ref, b, "mlp " + what)


@pytest.mark.timeout(600)
def test_prefill_layer_t2048(wl, orc):
    run_layer(wl, orc, inputs.GEMMA3_1B, 32, 2048, 0, None)


@pytest.mark.parametrize("r", [4, 16, 32])
def test_batched_decode_layer_t32(wl, orc, r):
    run_layer(wl, orc, inputs.GEMMA3_1B, r, 32, 0, 30)


@pytest.mark.parametrize("r", [4, 32])
def test_decode_layer_t1(wl, orc, r):
    run_layer(wl, orc, inputs.GEMMA3_1B, r, 1, 0, 0)


@pytest.mark.timeout(600)
def test_large_layer_t1(wl, orc):
    run_layer(wl, orc, inputs.LARGE_5376, 32, 1, 1, 0, w0_std=0.01)


@pytest.mark.timeout(900)
def test_large_layer_t512(wl, orc):
    run_layer(wl, orc, inputs.LARGE_5376, 32, 512, 1, None, w0_std=0.01)


@pytest.mark.parametrize("regime", [0, 1, 2, 4])
def test_shared_w0_layers_t32(wl, orc, regime):
    # G = 1: two layers alias one W0 per family (the same device tensor); each
    # layer keeps its own s, U, V. Every projection of both layers, every
    # element, in each regime that applies at T = 32.
    g = torch.Generator().manual_seed(7)
    dims = inputs.GEMMA3_1B
    lays = inputs.layers(g, dims, 32, 2, 1)
    assert lays[0]["gate"]["W0"] is lays[1]["gate"]["W0"]
    acts = inputs.layer_inputs(g, dims, 32)
    w0 = {f: lays[0][f]["W0"].to(DEV) for f in inputs.FAMILIES}
    prev = wl.set_regime(regime)
    try:
        for li, lay in enumerate(lays):
            dl = {f: dict(wl.theta_to(lay[f], DEV), W0=w0[f]) for f in inputs.FAMILIES}
            y_qkv = wl.wl_qkv_fused(dl["q"], dl["k"], dl["v"], acts["x_attn"].to(DEV))
            y_o = wl.wl_linear(dl["o"], acts["x_o"].to(DEV))
            y_mlp = wl.wl_mlp_fused(dl["gate"], dl["up"], dl["down"], acts["x_mlp"].to(DEV))
            torch.cuda.synchronize()
            what = f"shared-W0 layer {li} regime {regime}"
            y_ref, b = orc.qkv(lay["q"], lay["k"], lay["v"], acts["x_attn"])
            check(y_qkv, y_ref, b, "qkv " + what)
            y_ref, b = orc.linear(lay["o"], acts["x_o"])
            check(y_o, y_ref, b, "o " + what)
            y_ref, b, _ = orc.mlp(lay["gate"], lay["up"], lay["down"], acts["x_mlp"])
            check(y_mlp, y_ref, b, "mlp " + what)
    finally:
        wl.set_regime(prev)


def test_weff_full_gate_shape(wl, orc):
    g = torch.Generator().manual_seed(11)
    th = inputs.theta(g, 1152, 6912, 32)
    w = wl.wl_materialize_weff(wl.theta_to(th, DEV))
    rows = sample_tokens(6912, 6, 12)
    sub = dict(th, W0=th["W0"][rows], s=th["s"][rows], U=th["U"][rows], d_out=len(rows))
    w_ref, b = orc.weff(sub)
    check(w[torch.tensor(rows, device=DEV)], w_ref, b, f"W_eff rows {rows}")
    assert np.isfinite(w.float().cpu().numpy()).all()
