"""The fp32 variant of every operation against the CPU oracle (binary32 element type).

Every call goes through the C ABI with fp32 thetas (dtype WL_DTYPE_F32). Random
cases must meet the fp32 bars of ``parity.check_f32`` (derived from fp32
accumulation error); small-integer cases, whose every partial sum is exact in
fp32, must match the oracle bit for bit. Both fp32 kernels run on the same
cases: the wave-per-row GEMV (a few tokens) and the matrix-core GEMM.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from linear_02_amd import inputs
from parity import check_exact, check_f32

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32 = torch.float32


@pytest.fixture(scope="module")
def wl():
    from linear_02_amd import build
    if not os.path.exists(build.LIBRARY):
        build.build()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from linear_02_amd import wl as mod
    return mod


@pytest.fixture(params=["gemv", "mfma"])
def regime(request, wl):
    prev = wl.set_regime({"gemv": 1, "mfma": 2}[request.param])
    yield request.param
    wl.set_regime(prev)


def gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed)


def dev(th: dict) -> dict:
    from linear_02_amd import wl as mod
    return mod.theta_to(th, DEV)


LINEAR_CASES = [
    # d_in, d_out, r, T
    (1152, 1152, 4, 1),
    (8, 1, 1, 1),
    (24, 7, 3, 3),
    (136, 129, 17, 5),
    (1160, 300, 64, 2),
    (6912, 1152, 32, 1),
    (264, 520, 0, 8),
    (520, 264, 32, 33),
    (1152, 1536, 16, 130),       # several token tiles, ragged tail
    (3080, 131, 8, 70),          # partial last 16-input step, odd outputs
]


@pytest.mark.parametrize("d_in,d_out,r,T", LINEAR_CASES)
def test_linear_f32(wl, orc, regime, d_in, d_out, r, T):
    g = gen(1000 + d_in + 7 * d_out + T)
    th = inputs.theta(g, d_in, d_out, r, dtype=F32)
    x = inputs.activations(g, T, d_in, dtype=F32)
    y_ref, bound = orc.linear(th, x)
    y = wl.wl_linear(dev(th), x.to(DEV))
    check_f32(y, y_ref, bound, d_in + r, f"linear f32 {d_in}->{d_out} r={r} T={T} {regime}")


@pytest.mark.parametrize("T", [1, 5, 40])
def test_qkv_f32(wl, orc, regime, T):
    g = gen(1100 + T)
    dims = inputs.GEMMA3_1B
    q = inputs.theta(g, dims["d_model"], dims["q"], 32, dtype=F32)
    k = inputs.theta(g, dims["d_model"], dims["kv"], 16, dtype=F32)
    v = inputs.theta(g, dims["d_model"], dims["kv"], 0, dtype=F32)
    x = inputs.activations(g, T, dims["d_model"], dtype=F32)
    y_ref, bound = orc.qkv(q, k, v, x)
    y = wl.wl_qkv_fused(dev(q), dev(k), dev(v), x.to(DEV))
    check_f32(y, y_ref, bound, dims["d_model"] + 32, f"qkv f32 T={T} {regime}")


@pytest.mark.parametrize("d_model,d_ff,r,T", [(1152, 6912, 32, 1), (264, 520, 16, 3), (264, 520, 32, 33),
                                              (1152, 6912, 4, 20)])
def test_mlp_f32(wl, orc, regime, d_model, d_ff, r, T):
    g = gen(1200 + d_ff + T)
    gate = inputs.theta(g, d_model, d_ff, r, dtype=F32)
    up = inputs.theta(g, d_model, d_ff, r, dtype=F32)
    down = inputs.theta(g, d_ff, d_model, r, dtype=F32)
    x = inputs.activations(g, T, d_model, dtype=F32)
    y_ref, bound, _ = orc.mlp(gate, up, down, x)
    y = wl.wl_mlp_fused(dev(gate), dev(up), dev(down), x.to(DEV))
    check_f32(y, y_ref, bound, d_model + d_ff + 2 * r + 8, f"mlp f32 {d_model}/{d_ff} r={r} T={T} {regime}")


@pytest.mark.parametrize("d_in,d_out,r", [(1152, 1152, 32), (264, 136, 17), (8, 1, 64), (1024, 200, 0)])
def test_weff_f32(wl, orc, d_in, d_out, r):
    g = gen(1300 + d_in + d_out + r)
    th = inputs.theta(g, d_in, d_out, r, dtype=F32)
    w_ref, bound = orc.weff(th)
    w = wl.wl_materialize_weff(dev(th))
    check_f32(w, w_ref, bound, r + 4, f"weff f32 {d_in}x{d_out} r={r}")


def _int_theta(g, d_in, d_out, r):
    return dict(W0=inputs.int_tensor(g, (d_out, d_in), -8, 8, dtype=F32),
                s=inputs.choice_tensor(g, (d_out,), [0.5, 1.0, 2.0, -1.0]),
                U=inputs.int_tensor(g, (d_out, r), -2, 2, dtype=F32),
                V=inputs.int_tensor(g, (d_in, r), -2, 2, dtype=F32), d_in=d_in, d_out=d_out, r=r)


@pytest.mark.parametrize("d_in,d_out,r,T", [(136, 129, 17, 5), (1152, 1152, 8, 3), (520, 264, 32, 40)])
def test_linear_f32_bit_exact_integers(wl, orc, regime, d_in, d_out, r, T):
    # Integers up to 8 (far beyond what bf16 would keep at these sums): every
    # partial sum is an exact fp32 value, so any summation order gives the oracle's bits.
    g = gen(1400 + d_in + T)
    th = _int_theta(g, d_in, d_out, r)
    x = inputs.int_tensor(g, (T, d_in), -8, 8, dtype=F32)
    y_ref, _ = orc.linear(th, x)
    assert np.abs(y_ref).max() < 2 ** 24
    check_exact(wl.wl_linear(dev(th), x.to(DEV)), y_ref, f"linear f32 integers {regime}")
    w_ref, _ = orc.weff(th)
    check_exact(wl.wl_materialize_weff(dev(th)), w_ref, "weff f32 integers")


def test_mlp_f32_bit_exact_integers(wl, orc, regime):
    # One-hot x, gate entries in {-12, 0, 12, 16}: tanh-GELU is exactly z or 0 there in
    # fp32 and fp64, so h and y are exact integers.
    g = gen(1500)
    d_model, d_ff, T = 264, 520, 6
    x = torch.zeros(T, d_model)
    for t in range(T):
        x[t, int(torch.randint(0, d_model, (1,), generator=g))] = 1.0
    gate = dict(W0=inputs.choice_tensor(g, (d_ff, d_model), [-12.0, 0.0, 12.0, 16.0], F32),
                s=None, U=None, V=None, d_in=d_model, d_out=d_ff, r=0)
    up = dict(W0=inputs.int_tensor(g, (d_ff, d_model), -300, 300, dtype=F32), s=None, U=None, V=None,
              d_in=d_model, d_out=d_ff, r=0)
    dW = torch.zeros(d_model, d_ff)
    for o in range(d_model):
        cols = torch.randperm(d_ff, generator=g)[:4]
        dW[o, cols] = inputs.choice_tensor(g, (4,), [-1.0, 1.0])
    down = dict(W0=dW, s=inputs.choice_tensor(g, (d_model,), [0.5, 1.0, 2.0]), U=None, V=None,
                d_in=d_ff, d_out=d_model, r=0)
    y_ref, _, h = orc.mlp(gate, up, down, x)
    assert np.abs(h).max() > 256      # values a bf16 h could not hold
    y = wl.wl_mlp_fused(dev(gate), dev(up), dev(down), x.to(DEV))
    check_exact(y, y_ref, f"mlp f32 integers {regime}")


def test_f32_repeats_bitwise(wl):
    g = gen(1600)
    dims = inputs.GEMMA3_1B
    lay = inputs.layer(g, dims, 32, dtype=F32)
    dl = {f: dev(lay[f]) for f in lay}
    for T in (1, 48):
        x = inputs.activations(g, T, dims["d_model"], dtype=F32).to(DEV)
        a = wl.wl_mlp_fused(dl["gate"], dl["up"], dl["down"], x)
        b = wl.wl_mlp_fused(dl["gate"], dl["up"], dl["down"], x)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_f32_dtype_mismatch_raises(wl):
    g = gen(1700)
    q = dev(inputs.theta(g, 64, 32, 4, dtype=F32))
    k = dev(inputs.theta(g, 64, 16, 4))
    v = dev(inputs.theta(g, 64, 16, 4, dtype=F32))
    x = inputs.activations(g, 2, 64, dtype=F32).to(DEV)
    with pytest.raises(wl.WlError) as e:
        wl.wl_qkv_fused(q, k, v, x)
    assert e.value.status == 1
