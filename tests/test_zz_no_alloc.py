"""wl_linear_static: wl_linear with the library's static workspace.

Called through the C ABI (the binding only marshals arguments) and compared
with wl_linear on a workspace of its own: the same kernels run, so the outputs
agree bit for bit; both are also checked against the oracle. Two calls in a
row, the second smaller, show that the array's kept contents (tickets and
tagged words of the first call) do not disturb the next; a call whose
workspace would exceed the array fails before launching anything.
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


# (d_in, d_out, r, T): each list is run in order, each call on the previous one's array
SEQUENCES = [
    [(1152, 6912, 32, 8), (1152, 1152, 32, 1)],   # decode GEMV passes of 8 tokens, then one token
    [(6912, 1152, 32, 48), (1152, 1152, 16, 3)],  # few-token path, then a three-token decode pass
    [(1152, 1152, 4, 4), (1152, 1152, 4, 2)],     # the same shape, fewer tokens
]


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_static_workspace_matches_linear(wl, orc, seq):
    g = torch.Generator().manual_seed(7100 + seq)
    for d_in, d_out, r, T in SEQUENCES[seq]:
        th = inputs.theta(g, d_in, d_out, r)
        x = inputs.activations(g, T, d_in)
        dth = wl.theta_to(th, DEV)
        xd = x.to(DEV)
        print(f"static workspace d_in={d_in} d_out={d_out} r={r} T={T}", flush=True)
        y_static = torch.empty(T, d_out, dtype=torch.bfloat16, device=DEV)
        wl.wl_linear_static(dth, xd, y=y_static)
        ws = wl.new_workspace(wl.workspace_bytes(wl.OP_LINEAR, [dth], T), DEV)
        y_own = wl.wl_linear(dth, xd, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(y_static.view(torch.int16), y_own.view(torch.int16)), \
            f"static workspace differs from an own workspace at d_in={d_in} d_out={d_out} T={T}"
        y_ref, bound = orc.linear(th, x)
        check(y_static, y_ref, bound, f"static workspace d_in={d_in} d_out={d_out} r={r} T={T}")


def test_static_workspace_rejects_larger_calls(wl):
    d_in, d_out, r, T = 6912, 1152, 32, 2048
    g = torch.Generator().manual_seed(7200)
    th = inputs.theta(g, d_in, d_out, r)
    assert wl.workspace_bytes(wl.OP_LINEAR, [th], T) > wl.STATIC_SCRATCH_BYTES
    dth = wl.theta_to(th, DEV)
    x = torch.zeros(T, d_in, dtype=torch.bfloat16, device=DEV)
    y = torch.full((T, d_out), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(wl.WlError) as err:
        wl.wl_linear_static(dth, x, y=y)
    assert err.value.status == wl.WL_ERR_WORKSPACE
    assert "static scratch" in str(err.value)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a rejected call wrote its output"
