"""The decode kernel's in-launch V^T x hand-off (one to four tokens per pass).

Producer workgroups of the projection's own launch compute the V^T x slices
and publish them through the workspace's sync area; the other workgroups wait
for them (bounded) or, when the wait runs out, compute every slice themselves.
All three routes must give the same bits: the hand-off, the forced fallback
(spin limit 0) and the separate V^T x launch (regime 3), and the hand-off must
also meet the oracle bar. The MLP cases here run as two launches (regime 5, and
regime 3 for the separate V^T x launches); the one-launch MLP has tests of its
own (test_gpu_mlp.py). The sync area is checked after the calls: every
ticket counter advanced by exactly 2^24 per in-launch launch, no fallback on a
quiet device, and one per projection workgroup when forced.
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
STRIDE = 1 << 24
COPIES = 64


@pytest.fixture(scope="module")
def wl():
    from linear_02_amd import build
    if not os.path.exists(build.LIBRARY):
        build.build()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from linear_02_amd import wl as mod
    return mod


def consumer_workgroups(d_in: int, rows: int) -> int:
    """Projection workgroups of one decode launch: rows per workgroup from the
    row segmentation of the input axis (4 waves, 1/2/4 segments per row)."""
    nch = d_in // 8
    nseg = 1 if nch <= 640 else 2 if nch <= 1280 else 4
    R = 2 if nseg == 1 and nch <= 256 else 1
    rows_g = (4 // nseg) * R
    return -(-rows // rows_g)


def sync_words(ws: torch.Tensor) -> np.ndarray:
    return ws[:4096].view(torch.int64).cpu().numpy()


FINAL_OFFSET = 4096 + 8 * 64 * 4 * 64 * 8    # complete V^T x words of the two-level hand-off


def final_tags(ws: torch.Tensor, n_items: int) -> np.ndarray:
    w = ws[FINAL_OFFSET:FINAL_OFFSET + 8 * n_items].view(torch.int64).cpu().numpy()
    return (w.view(np.uint64) >> np.uint64(32)).astype(np.int64)


def slices(d_in: int) -> int:
    """Slices of the input axis: about 128 inputs each, at most 64, 8-aligned."""
    S = min(-(-d_in // 128), 64)
    slice_len = -(-(-(-d_in // S)) // 8) * 8
    return -(-d_in // slice_len)


def two_level(d_in: int, rows: int, T: int, sum_r: int) -> bool:
    """The plan's choice: two levels once projection workgroups x slices exceeds 4096."""
    return consumer_workgroups(d_in, rows) * slices(d_in) > 4096


# op, shapes, ranks: one and two levels, ragged and tiny grids, ranks 1 to 64,
# children without the low-rank term, the most producers one launch takes.
CASES = [
    ("linear", (1152, 1152), (32,)),
    ("linear", (6912, 1152), (32,)),          # 54 slices, rows in two segments
    ("linear", (136, 129), (17,)),            # ragged; grid below 64 workgroups
    ("linear", (8, 1), (1,)),                 # smallest: one producer, one consumer
    ("linear", (16384, 64), (64,)),           # 64 slices of 256 inputs, rank 64
    ("qkv", (1152, 1024, 256, 256), (32, 32, 32)),
    ("qkv", (1152, 256, 128, 128), (16, 0, 64)),   # a child without the low-rank term
    ("qkv", (16384, 64, 64, 64), (64, 64, 64)),    # 192 producers, the most one launch takes
    ("mlp", (1152, 6912), (32, 32, 32)),
    ("mlp", (1152, 6912), (0, 8, 4)),               # gate without the low-rank term
]


def make_case(op: str, shape: tuple, ranks: tuple, T: int, seed: int):
    g = torch.Generator().manual_seed(seed)
    if op == "linear":
        d_in, d_out = shape
        ths = [inputs.theta(g, d_in, d_out, ranks[0])]
        projs = [(d_in, d_out)]
    elif op == "qkv":
        d_in = shape[0]
        ths = [inputs.theta(g, d_in, d, r) for d, r in zip(shape[1:], ranks)]
        projs = [(d_in, sum(shape[1:]))]
    else:
        d, ff = shape
        ths = [inputs.theta(g, d, ff, ranks[0]), inputs.theta(g, d, ff, ranks[1]),
               inputs.theta(g, ff, d, ranks[2])]
        projs = [(d, ff), (ff, d)]
    x = inputs.activations(g, T, ths[0]["d_in"])
    return ths, x, projs


def run(wl, op, dths, xd, ws):
    if op == "linear":
        return wl.wl_linear(dths[0], xd, ws=ws)
    if op == "qkv":
        return wl.wl_qkv_fused(*dths, xd, ws=ws)
    return wl.wl_mlp_fused(*dths, xd, ws=ws)


def oracle(op, ths, x):
    from oracle.oracle import default
    orc = default()
    if op == "linear":
        return orc.linear(ths[0], x)
    if op == "qkv":
        return orc.qkv(*ths, x)
    y, b, _ = orc.mlp(*ths, x)
    return y, b


@pytest.mark.parametrize("T", [1, 2, 3, 4])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_handoff_fallback_and_separate_launch_agree(wl, case, T):
    op, shape, ranks = CASES[case]
    ths, x, projs = make_case(op, shape, ranks, T, seed=9100 + 10 * case + T)
    dths = [wl.theta_to(th, DEV) for th in ths]
    xd = x.to(DEV)
    wop = {"linear": wl.OP_LINEAR, "qkv": wl.OP_QKV, "mlp": wl.OP_MLP}[op]
    ws = wl.new_workspace(wl.workspace_bytes(wop, dths, T), DEV)
    print(f"hand-off case {op} {shape} r={ranks} T={T}", flush=True)
    in_launch = 5 if op == "mlp" else 1    # the MLP as two launches

    prev = wl.set_regime(3)
    try:
        y_sep = run(wl, op, dths, xd, ws).clone()
        torch.cuda.synchronize()
        assert not sync_words(ws).any(), "the separate V^T x launch touched the sync area"
        wl.set_regime(in_launch)
        reps = 3
        for _ in range(reps):
            y_inl = run(wl, op, dths, xd, ws).clone()
        torch.cuda.synchronize()
        words = sync_words(ws)
        launches = len(projs) * reps
        assert (words[:COPIES] == launches * STRIDE).all(), f"ticket counters {sorted(set(words[:COPIES]))}"
        assert words[511] == 0, f"{words[511]} workgroups stopped waiting on a quiet device"
        if op != "mlp":
            # Two levels leave the complete V^T x, tagged with the last launch's tag
            # (generation + 1 = launches), in the sync area; one level leaves it untouched.
            n_items = T * sum(ranks)
            tags = final_tags(ws, n_items)
            if two_level(projs[0][0], projs[0][1], T, sum(ranks)):
                assert (tags == launches).all(), f"complete V^T x tags {sorted(set(tags))}"
            else:
                assert not tags.any()

        spin = wl.set_spin_limit(0)
        try:
            y_fb = run(wl, op, dths, xd, ws).clone()
        finally:
            wl.set_spin_limit(spin)
        torch.cuda.synchronize()
        words = sync_words(ws)
        assert (words[:COPIES] == (launches + len(projs)) * STRIDE).all()
        expect_fb = sum(consumer_workgroups(d_in, rows) for d_in, rows in projs)
        assert words[511] == expect_fb == wl.fallback_count(ws)
    finally:
        wl.set_regime(prev)

    assert torch.equal(y_inl, y_sep), "hand-off and separate V^T x launch differ"
    assert torch.equal(y_fb, y_sep), "fallback and separate V^T x launch differ"
    y_ref, bound = oracle(op, ths, x)
    check(y_inl, y_ref, bound, f"{op} {shape} r={ranks} T={T}")


def test_sync_area_survives_workspace_sharing(wl):
    """Calls of every regime on one workspace, interleaved: the counters keep
    advancing in step (the other regimes leave the sync area alone), and each
    hand-off result still equals the separate launch's."""
    g = torch.Generator().manual_seed(9300)
    th = wl.theta_to(inputs.theta(g, 1152, 1152, 32), DEV)
    xs = [inputs.activations(g, T, 1152).to(DEV) for T in (1, 2, 40, 300, 1)]
    need = max(wl.workspace_bytes(wl.OP_LINEAR, [th], x.shape[0]) for x in xs)
    ws = wl.new_workspace(need, DEV)
    prev = wl.set_regime(0)
    try:
        outs = [wl.wl_linear(th, x, ws=ws).clone() for x in xs]
        wl.set_regime(3)
        refs = [wl.wl_linear(th, x, ws=ws).clone() for x in xs]
    finally:
        wl.set_regime(prev)
    torch.cuda.synchronize()
    words = sync_words(ws)
    assert (words[:COPIES] == 3 * STRIDE).all()   # T = 1, 2, 1 took the hand-off
    assert words[511] == 0
    for T, a, b in zip((1, 2, 40, 300, 1), outs, refs):
        if T <= 2:
            assert torch.equal(a, b), f"T={T}"
