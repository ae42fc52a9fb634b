"""The largest tensors the ABI accepts, on sampled outputs.

W0 with just under 2^31 elements (the ABI's limit per tensor), the widest
input the decode kernel takes (32768) and one input past it (which the
matrix-core path then serves), the maximum rank 64, bf16 and fp32. The weights
are deterministic integer patterns scaled by a power of two, filled on the
device row block by row block; the oracle computes the sampled output rows one
by one from the same values copied back.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from linear_02_amd import inputs
from parity import check, check_f32

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LIMIT = 1 << 31


@pytest.fixture(scope="module")
def wl():
    from linear_02_amd import build
    if not os.path.exists(build.LIBRARY):
        build.build()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from linear_02_amd import wl as mod
    return mod


def pattern(rows: int, cols: int, dtype, a: int, b: int, m: int, scale: float) -> torch.Tensor:
    """W[i][j] = ((a i + b j) mod m - m // 2) * scale, built on the device in row blocks."""
    out = torch.empty(rows, cols, dtype=dtype, device=DEV)
    col = torch.arange(cols, device=DEV, dtype=torch.int64)[None, :]
    for r0 in range(0, rows, 2048):
        r1 = min(rows, r0 + 2048)
        row = torch.arange(r0, r1, device=DEV, dtype=torch.int64)[:, None]
        out[r0:r1] = (((a * row + b * col) % m - m // 2).to(torch.float32) * scale).to(dtype)
    return out


def sampled_check(orc, th_dev: dict, x_host: torch.Tensor, y: torch.Tensor, rows: list, dtype, what: str):
    r = th_dev["r"]
    small = dict(W0=th_dev["W0"][rows].cpu(), s=th_dev["s"][rows].cpu(),
                 U=th_dev["U"][rows].cpu() if r else None, V=th_dev["V"].cpu() if r else None,
                 d_in=th_dev["d_in"], d_out=len(rows), r=r)
    y_ref, bound = orc.linear(small, x_host)
    got = y[:, rows]
    if dtype == torch.float32:
        check_f32(got, y_ref, bound, th_dev["d_in"] + r, what)
    else:
        check(got, y_ref, bound, what)


@pytest.mark.parametrize("dtype,d_in,d_out,T", [
    (torch.bfloat16, 32768, 65535, 1),      # widest decode input, W0 at 2^31 - 32768 elements
    (torch.bfloat16, 32768, 65535, 8),      # and eight tokens in one pass
    (torch.bfloat16, 32776, 65519, 3),      # past the decode kernel's width: matrix cores
    (torch.float32, 32768, 65535, 1),
    (torch.float32, 32768, 65535, 20),
])
def test_largest_weight(wl, orc, dtype, d_in, d_out, T):
    assert d_in * d_out < LIMIT
    g = torch.Generator().manual_seed(2000 + T)
    r = 64
    W0 = pattern(d_out, d_in, dtype, 7, 13, 17, 2.0 ** -6)
    s = (1 + 0.01 * torch.randn(d_out, generator=g)).to(DEV)
    U = (0.01 * torch.randn(d_out, r, generator=g)).to(dtype).to(DEV)
    V = (0.01 * torch.randn(d_in, r, generator=g)).to(dtype).to(DEV)
    x_host = inputs.activations(g, T, d_in, dtype=dtype)
    th = dict(W0=W0, s=s, U=U, V=V, d_in=d_in, d_out=d_out, r=r)
    y = wl.wl_linear(th, x_host.to(DEV))
    torch.cuda.synchronize()
    rows = [0, 1, 2, 31, 32, 4095, 12345, 32767, 32768, 40000, d_out - 33, d_out - 2, d_out - 1]
    sampled_check(orc, th, x_host, y, rows, dtype, f"largest W0 {dtype} {d_out}x{d_in} T={T}")
    del W0, y
    torch.cuda.empty_cache()


def test_largest_weff(wl, orc):
    d_in, d_out, r = 32768, 65535, 64
    g = torch.Generator().manual_seed(2100)
    W0 = pattern(d_out, d_in, torch.bfloat16, 5, 11, 13, 2.0 ** -5)
    s = (1 + 0.01 * torch.randn(d_out, generator=g)).to(DEV)
    U = (0.01 * torch.randn(d_out, r, generator=g)).to(torch.bfloat16).to(DEV)
    V = (0.01 * torch.randn(d_in, r, generator=g)).to(torch.bfloat16).to(DEV)
    th = dict(W0=W0, s=s, U=U, V=V, d_in=d_in, d_out=d_out, r=r)
    w = wl.wl_materialize_weff(th)
    torch.cuda.synchronize()
    rows = [0, 7, 32768, d_out - 1]
    small = dict(W0=W0[rows].cpu(), s=s[rows].cpu(), U=U[rows].cpu(), V=V.cpu(), d_in=d_in, d_out=len(rows), r=r)
    w_ref, bound = orc.weff(small)
    check(w[rows], w_ref, bound, "largest W_eff")
    del W0, w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [3, 4])
def test_widest_input_staged_x(wl, orc, T):
    # Passes of 3 and 4 tokens stage each producer's x slice in LDS; at d_in =
    # 32768 the slice is its longest (512 inputs). The in-launch hand-off, its
    # forced fallback (spin limit 0) and the separate V^T x launch (regime 3)
    # agree bit for bit, and sampled rows match the oracle.
    d_in, d_out, r = 32768, 65535, 64
    g = torch.Generator().manual_seed(2200 + T)
    W0 = pattern(d_out, d_in, torch.bfloat16, 7, 13, 17, 2.0 ** -6)
    s = (1 + 0.01 * torch.randn(d_out, generator=g)).to(DEV)
    U = (0.01 * torch.randn(d_out, r, generator=g)).to(torch.bfloat16).to(DEV)
    V = (0.01 * torch.randn(d_in, r, generator=g)).to(torch.bfloat16).to(DEV)
    x_host = inputs.activations(g, T, d_in)
    th = dict(W0=W0, s=s, U=U, V=V, d_in=d_in, d_out=d_out, r=r)
    xd = x_host.to(DEV)
    prev = wl.set_regime(1)
    try:
        y_hand = wl.wl_linear(th, xd).clone()
        spin = wl.set_spin_limit(0)
        try:
            y_fb = wl.wl_linear(th, xd).clone()
        finally:
            wl.set_spin_limit(spin)
        wl.set_regime(3)
        y_sep = wl.wl_linear(th, xd).clone()
        torch.cuda.synchronize()
    finally:
        wl.set_regime(prev)
    assert torch.equal(y_hand.view(torch.int16), y_fb.view(torch.int16)), "forced fallback differs"
    assert torch.equal(y_hand.view(torch.int16), y_sep.view(torch.int16)), "separate V^T x launch differs"
    rows = [0, 1, 511, 512, 32767, d_out - 1]
    sampled_check(orc, th, x_host, y_hand, rows, torch.bfloat16, f"widest input T={T}")
    del W0, y_hand, y_fb, y_sep
    torch.cuda.empty_cache()
