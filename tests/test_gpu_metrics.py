"""Reconstruction fidelity on the GPU: wl_relative_frobenius_error against the
oracle's relative Frobenius error ("What weightless inference costs",
"Reconstruction fidelity"), on the same bf16 values.

Both sides accumulate in fp64 in different orders, so they agree to about 1e-13
relative; the closed forms (R = W, R = 2W, W = 0) are exact on both.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

from linear_02_amd import inputs
from parity import to_f64

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


def bf16(g, n, std):
    return (std * torch.randn(n, generator=g)).to(torch.bfloat16)


@pytest.mark.parametrize("n", [1, 7, 8, 1000, 65536 + 5, 6912 * 1152])
def test_matches_oracle(wl, orc, n):
    g = torch.Generator().manual_seed(700 + n % 97)
    W = bf16(g, n, 0.02)
    R = (W.float() + bf16(g, n, 0.001).float()).to(torch.bfloat16)
    got = wl.relative_frobenius_error(W.to(DEV), R.to(DEV))
    ref = orc.rel_frob(to_f64(W), to_f64(R))
    assert math.isclose(got, ref, rel_tol=1e-12, abs_tol=0.0), (got, ref)
    # the same call twice gives the same bits
    assert wl.relative_frobenius_error(W.to(DEV), R.to(DEV)) == got


def test_closed_forms(wl):
    g = torch.Generator().manual_seed(5)
    W = bf16(g, 4099, 1.0).to(DEV)
    assert wl.relative_frobenius_error(W, W) == 0.0
    assert wl.relative_frobenius_error(W, (2 * W.float()).to(torch.bfloat16)) == 1.0   # doubling is exact
    Z = torch.zeros(4099, dtype=torch.bfloat16, device=DEV)
    assert wl.relative_frobenius_error(Z, Z) == 0.0
    assert wl.relative_frobenius_error(Z, W) == float("inf")


def test_weff_fidelity_against_dense_weight(wl, orc):
    # A theta's W_eff against the weight it reconstructs: here the reconstructed
    # weight is the fp64 oracle W_eff rounded to bf16, so the error is the bf16
    # rounding of W_eff (both sides see the same two bf16 tensors).
    g = torch.Generator().manual_seed(11)
    th = inputs.theta(g, 1152, 1152, 32)
    w_gpu = wl.wl_materialize_weff(wl.theta_to(th, DEV))
    w_ref, _ = orc.weff(th)
    W = torch.from_numpy(w_ref).to(torch.bfloat16)
    got = wl.relative_frobenius_error(W.to(DEV), w_gpu)
    ref = orc.rel_frob(to_f64(W), to_f64(w_gpu))
    assert math.isclose(got, ref, rel_tol=1e-12, abs_tol=1e-300)
    assert got < 2e-3
