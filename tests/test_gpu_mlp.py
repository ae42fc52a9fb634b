"""The MLP at decode sizes in one launch (one to four tokens per pass).

The launch splits the down projection along its input axis: each slice
workgroup forms h for its rows of the intermediate axis and the slice's share
of every down output, and groups of outputs are added over the slices in a
fixed order. Checked here against the oracle on shapes that reach one, two, four
and eight workgroups per slice, ragged slices (a part of the last slice empty)
and output groups, d_out != d_model, down ranks held as whole 16-byte pieces or
as single entries, no low-rank term, and s = None; bit for bit on integer cases; and bit for bit against its own forced
fallback (spin limit 0: every workgroup computes the gate/up V^T x itself and
every slice's workgroups compute each other's h rows, and every reduction
recomputes every slice's share). The ticket counters show that
the one-launch kernel ran: exactly one launch per pass of tokens.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from linear_02_amd import inputs
from parity import check, check_exact

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
    prev = mod.set_regime(1)
    yield mod
    mod.set_regime(prev)


def tokens_per_pass(T: int) -> int:
    tt = 1
    while tt < T and tt < 8:
        tt *= 2
    return tt


def slice_workgroups(d_ff: int, d_out: int, r_down: int) -> int:
    """Workgroups of the one-launch plan besides the producers (slices of 64
    intermediate rows x parts per slice), or 0 when the shape takes two launches."""
    if r_down % 8 != 0 and r_down >= 8:
        return 0
    n_slices = -(-d_ff // 64)
    if n_slices > 256:
        return 0
    for parts in (1, 2, 4, 8):
        if -(-d_out // parts) <= 18 * 32 and n_slices * parts <= 256:
            return n_slices * parts
    return 0


# d_model, d_ff, d_out, (r_gate, r_up, r_down), s present
CASES = [
    (1152, 6912, 1152, (32, 32, 32), True),    # the Gemma-3-1B-shaped MLP: 216 slices of 32
    (1152, 6912, 1152, (4, 4, 4), True),
    (1152, 6912, 1152, (0, 8, 4), True),       # gate without the low-rank term
    (1152, 6912, 1152, (0, 0, 0), True),       # no producers at all
    (1152, 6912, 1152, (32, 32, 32), False),   # s = None everywhere
    (264, 1000, 264, (16, 16, 3), True),       # ragged last slice (8 wide), down rank as entries
    (136, 520, 100, (17, 9, 24), True),        # d_out 100: ragged output group; d_model 136
    (1152, 64, 1152, (8, 8, 8), True),         # one slice, two workgroups
    (512, 16384, 512, (32, 32, 40), True),     # 256 slices of one workgroup, down rank 40
    (256, 8192, 256, (8, 8, 64), True),        # one workgroup per slice, down rank 64
    (2048, 2048, 2304, (32, 32, 32), True),    # four workgroups per slice; long gate/up rows
    (1024, 1032, 4096, (16, 16, 16), True),    # eight workgroups per slice; last slice 8 rows wide
    (4096, 2048, 1024, (32, 32, 32), True),    # 32 V^T x slices: the words are read after the stream
]


def make(case: int, T: int, seed: int):
    d_model, d_ff, d_out, (rg, ru, rd), with_s = CASES[case]
    g = torch.Generator().manual_seed(seed)
    gate = inputs.theta(g, d_model, d_ff, rg)
    up = inputs.theta(g, d_model, d_ff, ru)
    down = inputs.theta(g, d_ff, d_out, rd)
    if not with_s:
        for th in (gate, up, down):
            th["s"] = None
    x = inputs.activations(g, T, d_model)
    return gate, up, down, x


def counters(ws: torch.Tensor) -> np.ndarray:
    return ws[:4096].view(torch.int64).cpu().numpy()


@pytest.mark.parametrize("T", [1, 2, 3, 4])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_one_launch_mlp_matches_oracle(wl, orc, case, T):
    d_model, d_ff, d_out, ranks, _ = CASES[case]
    assert slice_workgroups(d_ff, d_out, ranks[2]) > 0
    gate, up, down, x = make(case, T, seed=5000 + 10 * case + T)
    dths = [wl.theta_to(th, DEV) for th in (gate, up, down)]
    ws = wl.new_workspace(wl.workspace_bytes(wl.OP_MLP, dths, T), DEV)
    print(f"one-launch mlp case {CASES[case]} T={T}", flush=True)
    y = wl.wl_mlp_fused(*dths, x.to(DEV), ws=ws)
    torch.cuda.synchronize()
    w = counters(ws)
    passes = -(-T // tokens_per_pass(T))
    assert (w[:COPIES] == passes * STRIDE).all(), f"ticket counters {sorted(set(w[:COPIES]))}"
    assert w[511] == 0, f"{w[511]} workgroups stopped waiting on a quiet device"
    y_ref, bound, _ = orc.mlp(gate, up, down, x)
    check(y, y_ref, bound, f"one-launch mlp {CASES[case]} T={T}")


@pytest.mark.parametrize("case,T", [(0, 1), (0, 4), (1, 3), (2, 2), (3, 1), (5, 2), (6, 4), (8, 1), (9, 1), (10, 3),
                                    (11, 2), (12, 1)])
def test_one_launch_mlp_fallback_is_bitwise(wl, case, T):
    gate, up, down, x = make(case, T, seed=5500 + 10 * case + T)
    dths = [wl.theta_to(th, DEV) for th in (gate, up, down)]
    xd = x.to(DEV)
    ws = wl.new_workspace(wl.workspace_bytes(wl.OP_MLP, dths, T), DEV)
    print(f"one-launch mlp fallback case {CASES[case]} T={T}", flush=True)
    y = wl.wl_mlp_fused(*dths, xd, ws=ws).clone()
    spin = wl.set_spin_limit(0)
    try:
        y_fb = wl.wl_mlp_fused(*dths, xd, ws=ws).clone()
    finally:
        wl.set_spin_limit(spin)
    y2 = wl.wl_mlp_fused(*dths, xd, ws=ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_fb.view(torch.int16)), "forced fallback differs"
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "not repeatable"
    w = counters(ws)
    passes = -(-T // tokens_per_pass(T))
    assert (w[:COPIES] == 3 * passes * STRIDE).all()
    d_model, d_ff, d_out, ranks, _ = CASES[case]
    expect_fb = passes * slice_workgroups(d_ff, d_out, ranks[2]) if ranks[0] + ranks[1] > 0 else 0
    assert w[511] == expect_fb, f"fallback count {w[511]}, expected {expect_fb}"


@pytest.mark.parametrize("T", [1, 3, 4])
def test_one_launch_mlp_integers_bit_exact(wl, orc, T):
    # One-hot x; gate entries in {-12, 0, 12, 16} (gelu_tanh exactly z or 0
    # there), up in [-2, 2] plus a 0/1 rank term, so |h| <= 48; down with two
    # +-1 per row, s in {1, 2} and a rank term of at most one h: every partial
    # sum is an integer below 256, exact in fp32 and bf16, whatever the order of
    # the additions.
    g = torch.Generator().manual_seed(990 + T)
    d_model, d_ff = 1152, 6912
    x = torch.zeros(T, d_model)
    for t in range(T):
        x[t, int(torch.randint(0, d_model, (1,), generator=g))] = 1.0
    x = x.to(torch.bfloat16)
    gate = dict(W0=inputs.choice_tensor(g, (d_ff, d_model), [-12.0, 0.0, 12.0, 16.0], torch.bfloat16),
                s=None, U=None, V=None, d_in=d_model, d_out=d_ff, r=0)
    Uu = torch.zeros(d_ff, 4)
    Uu[torch.randperm(d_ff, generator=g)[:50], 0] = 1.0
    Vu = torch.zeros(d_model, 4)
    Vu[:, 0] = inputs.choice_tensor(g, (d_model,), [0.0, 1.0])
    up = dict(W0=inputs.int_tensor(g, (d_ff, d_model), -2, 2), s=None, U=Uu.to(torch.bfloat16),
              V=Vu.to(torch.bfloat16), d_in=d_model, d_out=d_ff, r=4)
    dW = torch.zeros(d_model, d_ff)
    for o in range(d_model):
        cols = torch.randperm(d_ff, generator=g)[:2]
        dW[o, cols] = inputs.choice_tensor(g, (2,), [-1.0, 1.0])
    Ud = torch.zeros(d_model, 8)
    Ud[torch.randperm(d_model, generator=g)[:40], 1] = 1.0
    Vd = torch.zeros(d_ff, 8)
    Vd[torch.randperm(d_ff, generator=g)[:1], 1] = 1.0
    down = dict(W0=dW.to(torch.bfloat16), s=inputs.choice_tensor(g, (d_model,), [1.0, 2.0]),
                U=Ud.to(torch.bfloat16), V=Vd.to(torch.bfloat16), d_in=d_ff, d_out=d_model, r=8)
    y_ref, _, _ = orc.mlp(gate, up, down, x)
    assert np.abs(y_ref).max() <= 256 and np.abs(y_ref).max() > 0
    assert np.all(y_ref == np.round(y_ref))
    dths = [wl.theta_to(th, DEV) for th in (gate, up, down)]
    ws = wl.new_workspace(wl.workspace_bytes(wl.OP_MLP, dths, T), DEV)
    y = wl.wl_mlp_fused(*dths, x.to(DEV), ws=ws)
    torch.cuda.synchronize()
    assert (counters(ws)[:COPIES] == STRIDE).all()   # one launch
    check_exact(y, y_ref, f"one-launch mlp integers T={T}")


def test_workspace_init_clears_foreign_data(wl, orc):
    # A workspace full of garbage (bytes that could read as tagged words of any
    # generation), prepared by wl_workspace_init, gives the oracle's result.
    gate, up, down, x = make(0, 1, seed=5900)
    dths = [wl.theta_to(th, DEV) for th in (gate, up, down)]
    need = wl.workspace_bytes(wl.OP_MLP, dths, 1)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=DEV)
    ws[:4096].view(torch.int64)[:] = 5   # small tags a near-fresh launch would use
    wl.workspace_init(ws)
    y = wl.wl_mlp_fused(*dths, x.to(DEV), ws=ws)
    torch.cuda.synchronize()
    assert (counters(ws)[:COPIES] == STRIDE).all()
    y_ref, bound, _ = orc.mlp(gate, up, down, x)
    check(y, y_ref, bound, "after wl_workspace_init on garbage")
