"""HIP path against the CPU oracle, element by element, on seeded inputs.

Every call goes through the C ABI (linear_02_amd.wl -> libwl.so). Floating-point
cases must meet relL2 <= 2e-3 and |err| <= 8e-3 * bound per element; cases with
small-integer inputs, whose every partial sum is exact in fp32 and whose outputs
are exact in bf16, must match bit for bit. All kernel regimes (wave-per-row GEMV
with V^T x in the same launch or in a launch of its own, matrix-core GEMM, the
few-token split path, and the decode MLP in one launch or as two) are run on
the same cases (a forced regime that does not apply to a case runs the
matrix-core GEMM).
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from linear_02_amd import inputs
from parity import check, check_exact, to_f64

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


@pytest.fixture(params=["gemv", "mfma", "gemv2", "skinny", "mlp2", "mfma_sep"])
def regime(request, wl):
    prev = wl.set_regime({"gemv": 1, "mfma": 2, "gemv2": 3, "skinny": 4, "mlp2": 5, "mfma_sep": 6}[request.param])
    yield request.param
    wl.set_regime(prev)


def gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed)


def dev(th: dict) -> dict:
    from linear_02_amd import wl as mod
    return mod.theta_to(th, DEV)


def no_s(th: dict) -> dict:
    out = dict(th)
    out["s"] = None
    return out


# -- wl_linear ------------------------------------------------------------------------------

LINEAR_CASES = [
    # d_in, d_out, r, T
    (1152, 1152, 4, 1),       # the single projection at decode
    (8, 1, 1, 1),             # smallest shapes
    (24, 7, 3, 3),
    (136, 129, 17, 5),        # ragged everywhere
    (1160, 300, 64, 2),       # maximum rank
    (1024, 1152, 32, 4),      # attention output projection
    (6912, 1152, 32, 1),      # MLP down at decode: sliced V^T x
    (1152, 6912, 32, 1),
    (264, 520, 0, 9),         # no low-rank term
    (520, 264, 32, 33),
    (1152, 1536, 16, 130),    # several token tiles with a ragged tail
    (1152, 1152, 32, 32),     # batched decode: one full 32-token block
    (6912, 1152, 32, 17),     # long input axis, many splits, ragged tokens
    (1024, 1152, 4, 64),      # two token blocks
    (136, 129, 17, 12),       # ragged rows and input axis
    (3080, 136, 8, 70),       # matrix cores: input axis split in two, partial last step
    (3080, 131, 8, 70),       # the same with an odd output count (scalar reduction)
    (3080, 136, 5, 70),       # split input axis, odd rank: the reduction's scalar U path
    (6912, 256, 32, 1024),    # input axis in 4 splits, the rank term in the reduction
    (16384, 128, 16, 512),    # 10 splits: the rank term stays in the GEMM epilogue
]


@pytest.mark.parametrize("d_in,d_out,r,T", LINEAR_CASES)
def test_linear_matches_oracle(wl, orc, regime, d_in, d_out, r, T):
    g = gen(1000 + d_in + 7 * d_out + 13 * r + T)
    th = inputs.theta(g, d_in, d_out, r)
    x = inputs.activations(g, T, d_in)
    y_ref, bound = orc.linear(th, x)
    y = wl.wl_linear(dev(th), x.to(DEV))
    torch.cuda.synchronize()
    check(y, y_ref, bound, f"linear {d_in}->{d_out} r={r} T={T} {regime}")


def test_linear_without_scale_is_unit_scale(wl, orc, regime):
    g = gen(7)
    th = no_s(inputs.theta(g, 264, 136, 8))
    x = inputs.activations(g, 6, 264)
    y_ref, bound = orc.linear(th, x)
    y = wl.wl_linear(dev(th), x.to(DEV))
    check(y, y_ref, bound, "s=None")


def test_linear_deterministic(wl, regime):
    g = gen(11)
    th = dev(inputs.theta(g, 1152, 1152, 32))
    x = inputs.activations(g, 17, 1152).to(DEV)
    a = wl.wl_linear(th, x)
    b = wl.wl_linear(th, x)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_linear_t0_is_noop(wl):
    th = dev(inputs.theta(gen(3), 64, 32, 4))
    y = wl.wl_linear(th, torch.empty(0, 64, dtype=torch.bfloat16, device=DEV))
    assert tuple(y.shape) == (0, 32)


def _int_theta(g, d_in, d_out, r, *, w_lo=-2, w_hi=2, w_density=1.0, u_per_row=None, v_density=1.0):
    W0 = inputs.int_tensor(g, (d_out, d_in), w_lo, w_hi, density=w_density)
    s = inputs.choice_tensor(g, (d_out,), [0.5, 1.0, 2.0, -1.0])
    U = inputs.int_tensor(g, (d_out, r), -1, 1)
    if u_per_row is not None and r > u_per_row:
        keep = torch.zeros(d_out, r)
        for o in range(d_out):
            keep[o, torch.randperm(r, generator=g)[:u_per_row]] = 1
        U = (U.float() * keep).to(torch.bfloat16)
    V = inputs.int_tensor(g, (d_in, r), -1, 1, density=v_density)
    return dict(W0=W0, s=s, U=U, V=V, d_in=d_in, d_out=d_out, r=r)


@pytest.mark.parametrize("d_in,d_out,r,T", [(16, 24, 4, 3), (8, 5, 1, 1), (16, 17, 3, 2)])
def test_linear_bit_exact_tiny_integers(wl, orc, regime, d_in, d_out, r, T):
    # |y| <= 2*16*4 + 4*16 = 192: exact in fp32 sums and in bf16.
    g = gen(d_in * 100 + d_out)
    th = _int_theta(g, d_in, d_out, r)
    x = inputs.int_tensor(g, (T, d_in), -2, 2)
    y_ref, _ = orc.linear(th, x)
    assert np.abs(y_ref).max() <= 256
    y = wl.wl_linear(dev(th), x.to(DEV))
    check_exact(y, y_ref, f"tiny integers {regime}")


@pytest.mark.parametrize("d_in,d_out,r,T", [
    (1152, 1152, 4, 1), (6912, 1152, 32, 3), (1152, 6912, 32, 1), (5376, 2048, 32, 2), (1152, 1536, 16, 40)])
def test_linear_bit_exact_full_shapes(wl, orc, regime, d_in, d_out, r, T):
    # x: 16 entries of +-1 per token; W0 in [-2, 2]; U at most 4 nonzeros per row:
    # |s m| <= 2*32, |sum U vtx| <= 4*16, so every value is an integer below 256.
    g = gen(d_in + d_out + r + T)
    th = _int_theta(g, d_in, d_out, r, u_per_row=4)
    x = inputs.sparse_pm1_rows(g, T, d_in, 16)
    y_ref, _ = orc.linear(th, x)
    assert np.abs(y_ref).max() <= 256
    y = wl.wl_linear(dev(th), x.to(DEV))
    check_exact(y, y_ref, f"integer {d_in}->{d_out} r={r} T={T} {regime}")


def test_passthrough_point(wl, orc, regime):
    # U = V = 0 and s = 1: the reconstruction is W0 itself ("Serve and generate
    # with weightless", the passthrough operating point).
    g = gen(5)
    th = inputs.theta(g, 1152, 1152, 4)
    th["U"] = torch.zeros_like(th["U"])
    th["V"] = torch.zeros_like(th["V"])
    th["s"] = torch.ones_like(th["s"])
    x = inputs.activations(g, 3, 1152)
    y_ref, bound = orc.linear(th, x)
    dense, dbound = orc.linear(dict(th, r=0, s=None), x)
    assert np.array_equal(y_ref, dense)
    y = wl.wl_linear(dev(th), x.to(DEV))
    y_dense = wl.wl_linear(dev(dict(th, r=0, s=None, U=None, V=None)), x.to(DEV))
    check(y, y_ref, bound, "passthrough")
    assert torch.equal(y.view(torch.int16), y_dense.view(torch.int16))


# -- wl_qkv_fused ---------------------------------------------------------------------------

@pytest.mark.parametrize("r,T", [(4, 1), (32, 1), (32, 33)])
def test_qkv_matches_oracle_and_separate_calls(wl, orc, regime, r, T):
    g = gen(200 + r + T)
    shapes = inputs.family_shapes(inputs.GEMMA3_1B)
    q, k, v = (inputs.theta(g, *shapes[f], r) for f in ("q", "k", "v"))
    x = inputs.activations(g, T, 1152)
    y_ref, bound = orc.qkv(q, k, v, x)
    dq, dk, dv = dev(q), dev(k), dev(v)
    xd = x.to(DEV)
    y = wl.wl_qkv_fused(dq, dk, dv, xd)
    check(y, y_ref, bound, f"qkv r={r} T={T} {regime}")
    sep = torch.cat([wl.wl_linear(t, xd) for t in (dq, dk, dv)], dim=1)
    assert torch.equal(y.view(torch.int16), sep.view(torch.int16))


def test_qkv_mixed_children(wl, orc, regime):
    g = gen(77)
    q = inputs.theta(g, 264, 200, 32)
    k = no_s(inputs.theta(g, 264, 24, 0))
    v = inputs.theta(g, 264, 136, 5)
    x = inputs.activations(g, 10, 264)
    y_ref, bound = orc.qkv(q, k, v, x)
    y = wl.wl_qkv_fused(dev(q), dev(k), dev(v), x.to(DEV))
    check(y, y_ref, bound, "qkv mixed")


# -- wl_mlp_fused ---------------------------------------------------------------------------

@pytest.mark.parametrize("d_model,d_ff,r,T", [
    (1152, 6912, 4, 1), (1152, 6912, 32, 1), (264, 520, 16, 3), (264, 520, 32, 33), (1152, 6912, 32, 32)])
def test_mlp_matches_oracle(wl, orc, regime, d_model, d_ff, r, T):
    g = gen(300 + d_ff + r + T)
    gate = inputs.theta(g, d_model, d_ff, r)
    up = inputs.theta(g, d_model, d_ff, r)
    down = inputs.theta(g, d_ff, d_model, r)
    x = inputs.activations(g, T, d_model)
    y_ref, bound, _ = orc.mlp(gate, up, down, x)
    y = wl.wl_mlp_fused(dev(gate), dev(up), dev(down), x.to(DEV))
    check(y, y_ref, bound, f"mlp {d_model}/{d_ff} r={r} T={T} {regime}")


def test_mlp_bit_exact_integers(wl, orc, regime):
    # x one-hot per token, gate entries in {-12, 0, 12, 16}: gelu_tanh is exactly
    # z for those positive values and exactly 0 for -12 and 0 in fp32 and fp64;
    # up in [-2, 2], down with at most four +-1 per row: every value is an exact
    # small integer.
    g = gen(99)
    d_model, d_ff, T = 264, 520, 5
    x = torch.zeros(T, d_model)
    for t in range(T):
        x[t, int(torch.randint(0, d_model, (1,), generator=g))] = 1.0
    x = x.to(torch.bfloat16)
    gate = dict(W0=inputs.choice_tensor(g, (d_ff, d_model), [-12.0, 0.0, 12.0, 16.0], torch.bfloat16),
                s=None, U=None, V=None, d_in=d_model, d_out=d_ff, r=0)
    up = dict(W0=inputs.int_tensor(g, (d_ff, d_model), -2, 2), s=None, U=None, V=None,
              d_in=d_model, d_out=d_ff, r=0)
    dW = torch.zeros(d_model, d_ff)
    for o in range(d_model):
        cols = torch.randperm(d_ff, generator=g)[:4]
        dW[o, cols] = inputs.choice_tensor(g, (4,), [-1.0, 1.0])
    down = dict(W0=dW.to(torch.bfloat16), s=inputs.choice_tensor(g, (d_model,), [0.5, 1.0, 2.0]),
                U=None, V=None, d_in=d_ff, d_out=d_model, r=0)
    y_ref, _, _ = orc.mlp(gate, up, down, x)
    assert np.abs(y_ref).max() <= 256 and np.abs(y_ref).max() > 0
    y = wl.wl_mlp_fused(dev(gate), dev(up), dev(down), x.to(DEV))
    check_exact(y, y_ref, f"mlp integers {regime}")


# -- wl_materialize_weff ----------------------------------------------------------------------

@pytest.mark.parametrize("d_in,d_out,r", [(1152, 1152, 32), (1152, 6912, 4), (264, 136, 17), (8, 1, 64)])
def test_weff_matches_oracle(wl, orc, d_in, d_out, r):
    g = gen(400 + d_in + d_out + r)
    th = inputs.theta(g, d_in, d_out, r)
    w_ref, bound = orc.weff(th)
    w = wl.wl_materialize_weff(dev(th))
    check(w, w_ref, bound, f"weff {d_out}x{d_in} r={r}")
    rel = orc.rel_frob(w_ref, to_f64(w))
    assert rel <= 2e-3


def test_weff_batch_equals_single_calls(wl, orc):
    """wl_materialize_weff_batch: the seven projections of a Gemma-3-1B-shaped
    layer plus ragged shapes, r = 0 with s = None, odd ranks and rank 64 (ten
    thetas: two launches), bit for bit the one-projection results, and one of
    them against the oracle."""
    g = gen(4100)
    sh = inputs.family_shapes(inputs.GEMMA3_1B)
    ths = [inputs.theta(g, *sh[f], 32) for f in ("q", "k", "v", "o", "gate", "up", "down")]
    ths += [inputs.theta(g, 264, 136, 17), no_s(inputs.theta(g, 136, 129, 0)), inputs.theta(g, 8, 1, 64)]
    dths = [dev(th) for th in ths]
    outs = wl.wl_materialize_weff_batch(dths)
    torch.cuda.synchronize()
    for j, (dth, w) in enumerate(zip(dths, outs)):
        single = wl.wl_materialize_weff(dth)
        assert torch.equal(w.view(torch.int16), single.view(torch.int16)), f"theta {j}"
    w_ref, bound = orc.weff(ths[7])
    check(outs[7], w_ref, bound, "weff batch 136x264 r=17")


def test_weff_passthrough_and_integers(wl, orc):
    g = gen(41)
    th = inputs.theta(g, 264, 136, 0)
    th["s"] = None
    w = wl.wl_materialize_weff(dev(th))
    assert torch.equal(w.cpu().view(torch.int16), th["W0"].view(torch.int16))
    ti = _int_theta(g, 264, 136, 8)
    w_ref, _ = orc.weff(ti)
    check_exact(wl.wl_materialize_weff(dev(ti)), w_ref, "weff integers")


def test_dense_comparator_on_weff(wl, orc, regime):
    # The precompute-outside path: materialize W_eff, then a plain product with it.
    g = gen(43)
    th = inputs.theta(g, 1152, 1152, 32)
    x = inputs.activations(g, 4, 1152)
    W_eff = wl.wl_materialize_weff(dev(th))
    dense = dict(W0=W_eff, s=None, U=None, V=None, d_in=1152, d_out=1152, r=0)
    y_ref, bound = orc.linear(dict(dense, W0=W_eff.cpu()), x)
    y = wl.wl_linear(dense, x.to(DEV))
    check(y, y_ref, bound, "dense W_eff")


# -- error handling on the device path ------------------------------------------------------

def test_small_workspace_raises_and_nothing_breaks(wl, orc):
    g = gen(45)
    th = inputs.theta(g, 1152, 1152, 32)
    x = inputs.activations(g, 1, 1152)
    dth, xd = dev(th), x.to(DEV)
    small = torch.zeros(256, dtype=torch.uint8, device=DEV)
    with pytest.raises(wl.WlError) as e:
        wl.wl_linear(dth, xd, ws=small)
    assert e.value.status == 4
    y_ref, bound = orc.linear(th, x)
    check(wl.wl_linear(dth, xd), y_ref, bound, "after error")


# -- the decode kernel's in-kernel V^T x handoff ----------------------------------------------

@pytest.mark.parametrize("op", ["qkv", "mlp"])
def test_decode_handoff_repeats_bitwise(wl, orc, op):
    # Hundreds of back-to-back launches with no host synchronization in between:
    # every result must carry the same bits as the first and meet the oracle.
    g = gen(600)
    dims = inputs.GEMMA3_1B
    lay = inputs.layer(g, dims, 32)
    x = inputs.activations(g, 1, dims["d_model"])
    dl = {f: dev(lay[f]) for f in lay}
    xd = x.to(DEV)
    n = 300
    if op == "qkv":
        out = torch.empty(n, dims["q"] + 2 * dims["kv"], dtype=torch.bfloat16, device=DEV)
        for i in range(n):
            wl.wl_qkv_fused(dl["q"], dl["k"], dl["v"], xd, y=out[i:i + 1])
        y_ref, bound = orc.qkv(lay["q"], lay["k"], lay["v"], x)
    else:
        out = torch.empty(n, dims["d_model"], dtype=torch.bfloat16, device=DEV)
        for i in range(n):
            wl.wl_mlp_fused(dl["gate"], dl["up"], dl["down"], xd, y=out[i:i + 1])
        y_ref, bound, _ = orc.mlp(lay["gate"], lay["up"], lay["down"], x)
    torch.cuda.synchronize()
    bits = out.view(torch.int16)
    same = (bits == bits[0:1]).all(dim=1)
    assert bool(same.all()), f"{int((~same).sum())} of {n} launches differ from the first"
    check(out[0:1], y_ref, bound, f"{op} repeated")
