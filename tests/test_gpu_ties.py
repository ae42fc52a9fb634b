"""Round-to-nearest-even at exact bf16 ties, on the GPU, in every regime.

The output cast ("In-kernel reconstruction", the custom-op path: accumulate in
float32, cast back to the output dtype) must round a value exactly halfway
between two bf16 neighbours to the one with an even last bit. Random inputs
almost never land on a tie, so these cases are built to: every product is exact
and every partial sum fits in 24 bits, so fp32 accumulation in any order gives
the exact value, and the cast alone decides. Rows take their small terms from
W0 or from the rank term, s is 1/2, 1 or 2, and each token scales x by a power
of two (ties stay ties). The expected bits are the oracle's exact result
rounded by its pinned RNE; a few rows are also checked against literal values
(1 + 2^-8 -> 1, 1 + 3 2^-8 -> 1 + 2^-6), and each case asserts that it holds
both kinds of tie. Covered: the linear and Q/K/V in every regime, the MLP's h
(gate 16, where GELU-tanh is exactly 16, times an up value at a tie), and W_eff.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from parity import check_exact

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (terms added in the sum, s); terms are bf16 values, the exact sum s * sum(terms)
# sits at, just above or just below a tie between bf16 neighbours.
PATTERNS = [
    ((1.0, 2.0**-8), 1.0),                  # 1 + 2^-8: halfway, to even -> 1
    ((1.0, 3 * 2.0**-8), 1.0),              # 1 + 3 2^-8: halfway, to even -> 1 + 2^-6
    ((-1.0, -2.0**-8), 1.0),                # -> -1
    ((-1.0, -3 * 2.0**-8), 1.0),            # -> -(1 + 2^-6)
    ((1.0, 2.0**-8, 2.0**-20), 1.0),        # just above the tie -> 1 + 2^-7
    ((1.0, 2.0**-8, -2.0**-20), 1.0),       # just below -> 1
    ((256.0, 1.0), 1.0),                    # 257: halfway between 256 and 258 -> 256
    ((256.0, 3.0), 1.0),                    # 259 -> 260
    ((2.0**-10, 2.0**-18), 1.0),            # small magnitude -> 2^-10
    ((0.5, 2.0**-9), 2.0),                  # s = 2: 1 + 2^-8 -> 1
    ((1.0, 3 * 2.0**-8), 0.5),              # s = 1/2: 1/2 + 3 2^-9 -> 1/2 + 2^-7
    ((1.5, 2.0**-8), 1.0),                  # 1.5 + 2^-8: halfway, even is 1.5 -> 1.5
    ((1.0 + 2.0**-7, 2.0**-8), 1.0),        # odd neighbour below -> 1 + 2^-6
]
N_TERMS = 3
RANK = 8


@pytest.fixture(scope="module")
def wl():
    from linear_02_amd import build
    if not os.path.exists(build.LIBRARY):
        build.build()
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    from linear_02_amd import wl as mod
    return mod


def tie_theta(d_in: int, d_out: int, offset: int = 0, use_s: bool = True) -> dict:
    """Row o takes pattern (o + offset) % len(PATTERNS). Even pattern rounds put
    every term in W0 (columns 0..2); odd ones put the first term in W0 and the
    others, times s, in the rank term (U[o][k] with V[k][k] = 1, so the rank
    term is sum_k U[o][k] x[k] and is not scaled by s). use_s False sets every
    s to 1 (the patterns' sums unscaled)."""
    W0 = torch.zeros(d_out, d_in)
    U = torch.zeros(d_out, RANK)
    V = torch.zeros(d_in, RANK)
    for k in range(N_TERMS):
        V[k, k] = 1.0
    s = torch.ones(d_out)
    for o in range(d_out):
        j = o + offset
        terms, so = PATTERNS[j % len(PATTERNS)]
        so = so if use_s else 1.0
        s[o] = so
        if (j // len(PATTERNS)) % 2 == 0:
            for k, v in enumerate(terms):
                W0[o, k] = v
        else:
            W0[o, 0] = terms[0]
            for k, v in enumerate(terms[1:], start=1):
                U[o, k] = so * v
    bf = torch.bfloat16
    for t in (W0, U, V):
        assert torch.equal(t.to(bf).float(), t)   # every entry is a bf16 value
    return dict(W0=W0.to(bf), s=s, U=U.to(bf), V=V.to(bf), d_in=d_in, d_out=d_out, r=RANK)


def tie_x(T: int, d_in: int) -> torch.Tensor:
    x = torch.zeros(T, d_in)
    for t in range(T):
        x[t, :N_TERMS] = 2.0 ** ((t % 5) - 2)
    return x.to(torch.bfloat16)


def rne_bits(orc, y: np.ndarray) -> np.ndarray:
    flat = [orc.bf16_rne(float(v)) for v in y.reshape(-1)]
    return np.array(flat, dtype=np.uint16).reshape(y.shape)


def bf16_of_bits(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def count_ties(y: np.ndarray) -> tuple[int, int]:
    """Exact ties in y (fp64) whose RNE keeps the lower / takes the upper neighbour
    in magnitude (normal range: quantum 2^(e - 8) in the binade [2^(e-1), 2^e))."""
    a = np.abs(y[np.isfinite(y) & (y != 0)])
    _, e = np.frexp(a)
    r = a / np.ldexp(1.0, e - 8)
    lo = np.floor(r)
    tie = (r - lo) == 0.5
    odd = lo[tie].astype(np.int64) % 2 == 1
    return int(np.sum(~odd)), int(np.sum(odd))


def expect_ties(orc, y_ref: np.ndarray, what: str) -> np.ndarray:
    down, up = count_ties(y_ref)
    assert down > 0 and up > 0, f"{what}: the case holds {down} ties to round down and {up} to round up"
    return bf16_of_bits(rne_bits(orc, y_ref))


REGIMES = [0, 1, 2, 3, 4, 5, 6]


@pytest.mark.parametrize("T", [1, 3, 32])
@pytest.mark.parametrize("regime", REGIMES)
def test_linear_rounds_ties_to_even(wl, orc, regime, T):
    th = tie_theta(1152, 1152)
    x = tie_x(T, 1152)
    y_ref, _ = orc.linear(th, x)
    want = expect_ties(orc, y_ref, "linear")
    # literal checks on rows with x = 1 (token 2): patterns 0 and 1 in W0
    if T > 2:
        assert want[2, 0] == 1.0 and want[2, 1] == 1 + 2.0**-6
    prev = wl.set_regime(regime)
    try:
        y = wl.wl_linear(wl.theta_to(th, DEV), x.to(DEV))
        torch.cuda.synchronize()
    finally:
        wl.set_regime(prev)
    check_exact(y, want, f"linear ties regime {regime} T={T}")


@pytest.mark.parametrize("regime", [2, 6])
def test_split_projection_rounds_ties_to_even(wl, orc, regime):
    """A projection whose input axis is split (6912 inputs, 256 outputs, T = 1024:
    four splits): the rank term added in the reduction (regime 2) or in split
    0's epilogue (regime 6), one rounding either way."""
    T = 1024
    th = tie_theta(6912, 256)
    x = tie_x(T, 6912)
    y_ref, _ = orc.linear(th, x)
    want = expect_ties(orc, y_ref, "split linear")
    prev = wl.set_regime(regime)
    try:
        y = wl.wl_linear(wl.theta_to(th, DEV), x.to(DEV))
        torch.cuda.synchronize()
    finally:
        wl.set_regime(prev)
    check_exact(y, want, f"split linear ties regime {regime}")


@pytest.mark.parametrize("T", [1, 4, 32])
@pytest.mark.parametrize("regime", REGIMES)
def test_qkv_rounds_ties_to_even(wl, orc, regime, T):
    q, k, v = tie_theta(1152, 1024, 0), tie_theta(1152, 256, 5), tie_theta(1152, 256, 9)
    x = tie_x(T, 1152)
    y_ref, _ = orc.qkv(q, k, v, x)
    want = expect_ties(orc, y_ref, "qkv")
    prev = wl.set_regime(regime)
    try:
        y = wl.wl_qkv_fused(*(wl.theta_to(t, DEV) for t in (q, k, v)), x.to(DEV))
        torch.cuda.synchronize()
    finally:
        wl.set_regime(prev)
    check_exact(y, want, f"qkv ties regime {regime} T={T}")


def mlp_ties(d_model: int, d_ff: int):
    """gate: 16 on column 0 (GELU-tanh(16) is exactly 16 in fp32 and fp64);
    up: tie patterns with s = 1 (so h = 16 u sits at the scaled tie); down:
    row o picks h[o] with weight 1 (its rank term has U = 0), so y = h."""
    bf = torch.bfloat16
    gate = dict(W0=torch.zeros(d_ff, d_model), s=None, U=None, V=None, d_in=d_model, d_out=d_ff, r=0)
    gate["W0"][:, 0] = 16.0
    gate["W0"] = gate["W0"].to(bf)
    up = tie_theta(d_model, d_ff, use_s=False)
    dW = torch.zeros(d_model, d_ff)
    for o in range(d_model):
        dW[o, o] = 1.0
    down = dict(W0=dW.to(bf), s=None, U=torch.zeros(d_model, 4, dtype=bf),
                V=torch.full((d_ff, 4), 0.5).to(bf), d_in=d_ff, d_out=d_model, r=4)
    return gate, up, down


@pytest.mark.parametrize("T", [1, 2, 4, 32])
@pytest.mark.parametrize("regime", REGIMES)
def test_mlp_h_rounds_ties_to_even(wl, orc, regime, T):
    d_model, d_ff = 1152, 6912
    gate, up, down = mlp_ties(d_model, d_ff)
    x = torch.zeros(T, d_model)
    x[:, :N_TERMS] = 1.0   # h = 16 u: the first token row holds the ties; all tokens alike
    x = x.to(torch.bfloat16)
    g_ref, _ = orc.linear(gate, x)
    assert np.all(g_ref == 16.0) and orc.gelu(16.0) == 16.0
    u_ref, _ = orc.linear(up, x)
    expect_ties(orc, 16.0 * u_ref, "mlp h")
    y_ref, _, h = orc.mlp(gate, up, down, x)
    assert bf16_of_bits(h[0, :2]).tolist() == [16.0, 16.0 * (1 + 2.0**-6)]
    assert np.array_equal(y_ref, bf16_of_bits(h[:, :d_model]))   # y = h exactly
    prev = wl.set_regime(regime)
    try:
        y = wl.wl_mlp_fused(*(wl.theta_to(t, DEV) for t in (gate, up, down)), x.to(DEV))
        torch.cuda.synchronize()
    finally:
        wl.set_regime(prev)
    check_exact(y, y_ref, f"mlp h ties regime {regime} T={T}")


def test_weff_rounds_ties_to_even(wl, orc):
    d_in, d_out = 1152, 1152
    bf = torch.bfloat16
    W0 = torch.zeros(d_out, d_in)
    U = torch.zeros(d_out, RANK)
    V = torch.zeros(d_in, RANK)
    s = torch.ones(d_out)
    V[:, 0] = torch.tensor([1.0, 0.5, 1.0, -1.0])[torch.arange(d_in) % 4]
    for o in range(d_out):
        terms, so = PATTERNS[o % len(PATTERNS)]
        W0[o, :] = terms[0]
        s[o] = so
        U[o, 0] = so * terms[1]   # column i: s a + s b V[i][0] (+ c below)
        if len(terms) > 2:
            U[o, 1] = so * terms[2]
            V[:, 1] = 1.0
    th = dict(W0=W0.to(bf), s=s, U=U.to(bf), V=V.to(bf), d_in=d_in, d_out=d_out, r=RANK)
    w_ref, _ = orc.weff(th)
    want = expect_ties(orc, w_ref, "W_eff")
    assert want[0, 0] == 1.0 and want[1, 0] == 1 + 2.0**-6
    w = wl.wl_materialize_weff(wl.theta_to(th, DEV))
    torch.cuda.synchronize()
    check_exact(w, want, "W_eff ties")
