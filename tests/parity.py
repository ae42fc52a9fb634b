"""Acceptance checks of HIP outputs against the CPU oracle.

Floating-point outputs pass when, over the whole output tensor of a call,
  relL2 = ||y_gpu - y_oracle||_2 / ||y_oracle||_2 <= 2e-3
and for every element
  |y_gpu - y_oracle| <= 8e-3 * bound,
bound being the oracle's magnitude bound |s| sum|W0 x| + sum|U vtx| (for W_eff:
|s W0| + sum|U V|). One bf16 rounding of the output costs at most half a unit in
the last of bf16's 8 significant bits, 2^-8 of |y| at worst, inside the
per-element bar since |y| <= bound; fp32 accumulation adds orders of magnitude
less.
relL2 is a statistical bar: a single correctly rounded bf16 value can carry a
relative error of 2^-8, above 2e-3, so for outputs of fewer than
MIN_REL_L2_ELEMS elements only the per-element bar applies. Over larger outputs
the rounding error averages to about 1.6e-3.
Integer-valued cases are compared bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

REL_L2 = 2e-3
ELEM = 8e-3
MIN_REL_L2_ELEMS = 256


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def check(y_gpu: torch.Tensor, y_ref: np.ndarray, bound: np.ndarray, what: str = "") -> dict:
    yg = to_f64(y_gpu).reshape(y_ref.shape)
    assert np.all(np.isfinite(yg)), f"{what}: non-finite output"
    diff = yg - y_ref
    nref = float(np.linalg.norm(y_ref))
    ndiff = float(np.linalg.norm(diff))
    rel = ndiff / nref if nref > 0 else (0.0 if ndiff == 0 else float("inf"))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, np.abs(diff) / bound, np.where(diff == 0, 0.0, np.inf))
    worst = float(ratio.max()) if ratio.size else 0.0
    if y_ref.size >= MIN_REL_L2_ELEMS:
        assert rel <= REL_L2, f"{what}: relL2 {rel:.3e} > {REL_L2}"
    assert worst <= ELEM, f"{what}: max |err|/bound {worst:.3e} > {ELEM} at {np.unravel_index(ratio.argmax(), ratio.shape)}"
    return dict(rel_l2=rel, max_err_over_bound=worst)


# fp32 variant. Sums of n products accumulated in fp32 (fused multiply-adds, any
# order) err by at most about n * 2^-24 of the sum of the magnitudes (Higham's
# gamma_n), so the per-element bar is (n + 4) * 2^-24 * bound, with n the longest
# accumulation of the call (d_in + r; the MLP adds the gate/up path, whose h
# errors feed the down projection). Rounding errors of random sign grow like
# sqrt(n) * 2^-24 of the output norm; relL2 <= 4 * sqrt(n) * 2^-24.
EPS32 = 2.0 ** -24


def check_f32(y_gpu: torch.Tensor, y_ref: np.ndarray, bound: np.ndarray, n_acc: int, what: str = "") -> dict:
    assert y_gpu.dtype == torch.float32, f"{what}: output is {y_gpu.dtype}"
    yg = y_gpu.detach().cpu().double().numpy().reshape(y_ref.shape)
    assert np.all(np.isfinite(yg)), f"{what}: non-finite output"
    diff = yg - y_ref
    nref = float(np.linalg.norm(y_ref))
    ndiff = float(np.linalg.norm(diff))
    rel = ndiff / nref if nref > 0 else (0.0 if ndiff == 0 else float("inf"))
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, np.abs(diff) / bound, np.where(diff == 0, 0.0, np.inf))
    worst = float(ratio.max()) if ratio.size else 0.0
    rel_bar, elem_bar = 4.0 * np.sqrt(n_acc) * EPS32, (n_acc + 4) * EPS32
    if y_ref.size >= MIN_REL_L2_ELEMS:
        assert rel <= rel_bar, f"{what}: relL2 {rel:.3e} > {rel_bar:.3e}"
    assert worst <= elem_bar, (f"{what}: max |err|/bound {worst:.3e} > {elem_bar:.3e} at "
                               f"{np.unravel_index(ratio.argmax(), ratio.shape)}")
    return dict(rel_l2=rel, max_err_over_bound=worst)


def check_exact(y_gpu: torch.Tensor, y_ref: np.ndarray, what: str = "") -> None:
    yg = to_f64(y_gpu).reshape(y_ref.shape)
    bad = np.argwhere(yg != y_ref)
    assert bad.size == 0, (f"{what}: {len(bad)} elements differ; first at {tuple(bad[0])}: "
                           f"gpu {yg[tuple(bad[0])]} vs oracle {y_ref[tuple(bad[0])]}")
