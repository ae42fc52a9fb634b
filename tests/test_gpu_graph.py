"""HIP graph capture of the library calls: every replay equals the eager result.

The benchmark replays captured graphs, so captured calls must keep producing
the eager bits: nothing in the captured work may depend on state left by the
host or by an earlier replay. Replays are interleaved with unrelated eager work
and synchronizations. T = 1 and 3 run the decode kernels, T = 40 the few-token
split path.
"""
from __future__ import annotations

import os

import pytest
import torch

from linear_02_amd import inputs

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


@pytest.mark.parametrize("T", [1, 3, 40])
def test_graph_replays_match_eager(wl, T):
    g = torch.Generator().manual_seed(500 + T)
    dims = inputs.GEMMA3_1B
    lay = {f: wl.theta_to(th, DEV) for f, th in inputs.layer(g, dims, 32).items()}
    acts = {k: v.to(DEV) for k, v in inputs.layer_inputs(g, dims, T).items()}
    ws_bytes = max(wl.workspace_bytes(wl.OP_QKV, [lay["q"], lay["k"], lay["v"]], T),
                   wl.workspace_bytes(wl.OP_MLP, [lay["gate"], lay["up"], lay["down"]], T))
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=DEV)
    y_qkv = torch.empty(T, dims["q"] + 2 * dims["kv"], dtype=torch.bfloat16, device=DEV)
    y_o = torch.empty(T, dims["d_model"], dtype=torch.bfloat16, device=DEV)
    y_m = torch.empty(T, dims["d_model"], dtype=torch.bfloat16, device=DEV)

    def step():
        wl.wl_qkv_fused(lay["q"], lay["k"], lay["v"], acts["x_attn"], y=y_qkv, ws=ws)
        wl.wl_linear(lay["o"], acts["x_o"], y=y_o, ws=ws)
        wl.wl_mlp_fused(lay["gate"], lay["up"], lay["down"], acts["x_mlp"], y=y_m, ws=ws)

    step()
    torch.cuda.synchronize()
    ref = [y.clone() for y in (y_qkv, y_o, y_m)]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for y in (y_qkv, y_o, y_m):
            y.fill_(7.0)
        scratch = torch.randn(1024, 1024, device=DEV) @ torch.randn(1024, 1024, device=DEV)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, y, r in zip(("qkv", "o", "mlp"), (y_qkv, y_o, y_m), ref):
            assert torch.equal(y.view(torch.int16), r.view(torch.int16)), f"replay {rep}: {name} differs"
        del scratch
    # eager again after the replays
    step()
    torch.cuda.synchronize()
    for y, r in zip((y_qkv, y_o, y_m), ref):
        assert torch.equal(y.view(torch.int16), r.view(torch.int16))
