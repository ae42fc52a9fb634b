"""The C-ABI library without a GPU: it loads, exports every declared symbol, and
rejects bad arguments on the host before touching the device.

Pointers below are fake addresses that are never dereferenced: every call here
fails validation (or is the T == 0 no-op) before anything reaches HIP.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(REPO, "include", "wl.h")
TEST_HEADER = os.path.join(REPO, "include", "wl_testing.h")


@pytest.fixture(scope="module")
def wl():
    from linear_02_amd import build
    if not os.path.exists(build.LIBRARY):
        build.build()
    from linear_02_amd import wl as mod
    return mod


def declared_functions(header: str = HEADER) -> list[str]:
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wl_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(wl):
    names = declared_functions() + declared_functions(TEST_HEADER)
    assert {"wl_linear", "wl_qkv_fused", "wl_mlp_fused", "wl_materialize_weff",
            "wl_workspace_bytes", "wl_workspace_init", "wl_sync_bytes"} <= set(names)
    # the switches for tests live in the test header only
    assert not {"wl_set_regime", "wl_set_spin_limit"} & set(declared_functions())
    assert {"wl_set_regime", "wl_set_spin_limit"} <= set(declared_functions(TEST_HEADER))
    out = subprocess.run(["nm", "-D", "--defined-only", wl.LIBRARY], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (wl_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for n in names:
        getattr(wl.lib, n)


def test_abi_version_and_status_strings(wl):
    assert wl.abi_version() == 6
    assert wl.lib.wl_status_str(0) == b"ok"
    assert wl.lib.wl_status_str(4) == b"workspace too small"
    assert wl.lib.wl_status_str(99) == b"unknown status"


A = 0x10000   # fake, 256-byte aligned device addresses
B = 0x20000000
C = 0x40000000
D = 0x60000000


def theta(W0=A, s=None, U=B, V=C, d_in=64, d_out=32, r=4):
    return wl_mod().Theta(W0, s, U, V, d_in, d_out, r)


def wl_mod():
    from linear_02_amd import wl as mod
    return mod


def call_linear(wl, th, x=D, y=D + 0x1000000, T=1, ws=D + 0x2000000, ws_bytes=1 << 30):
    p = None if th is None else ctypes.byref(th)
    return wl.lib.wl_linear(p, x, y, T, ws, ws_bytes, None)


@pytest.mark.parametrize("case,status", [
    (dict(d_in=60), 1),            # not a multiple of 8
    (dict(d_in=0), 1),
    (dict(d_out=0), 1),
    (dict(r=-1), 1),
    (dict(r=65), 2),               # above the supported rank
    (dict(W0=None), 1),
    (dict(W0=A + 8), 1),           # misaligned
    (dict(U=None), 1),
    (dict(V=B + 2), 1),
    (dict(s=A + 2), 1),
])
def test_linear_rejects_bad_theta(wl, case, status):
    assert call_linear(wl, theta(**case)) == status
    assert wl.lib.wl_last_error() != b""


def test_tensor_size_limit(wl):
    # W0 of exactly 2^31 elements is one too many; 2^31 - 32768 is accepted (the
    # call then fails only on the fake workspace size).
    assert call_linear(wl, theta(d_in=32768, d_out=65536)) == 1
    assert b"2^31" in wl.lib.wl_last_error()
    assert call_linear(wl, theta(d_in=32768, d_out=65535), ws_bytes=0) == 4


def test_linear_rejects_null_theta_and_io(wl):
    assert call_linear(wl, None) == 1
    assert call_linear(wl, theta(), x=None) == 1
    assert call_linear(wl, theta(), y=None) == 1
    assert call_linear(wl, theta(), x=D + 4) == 1
    assert call_linear(wl, theta(), T=-1) == 1


def test_r0_needs_no_factors(wl):
    th = theta(U=None, V=None, r=0)
    assert call_linear(wl, th, T=0) == 0


def test_t0_is_a_noop(wl):
    assert call_linear(wl, theta(), x=None, y=None, T=0, ws=None, ws_bytes=0) == 0
    assert wl.lib.wl_last_error() == b""


def test_workspace_checks(wl):
    th = theta()
    arr = (ctypes.POINTER(wl.Theta) * 1)(ctypes.pointer(th))
    need = wl.lib.wl_workspace_bytes(0, arr, 1, 1)
    assert need > 0 and need % 256 == 0
    assert call_linear(wl, th, ws_bytes=need - 1) == 4
    assert b"workspace" in wl.lib.wl_last_error()
    assert call_linear(wl, th, ws=None, ws_bytes=need) == 1
    assert call_linear(wl, th, ws=D + 0x2000010, ws_bytes=need) == 1   # misaligned


def test_workspace_bytes_grows_with_tokens_and_rejects_bad_args(wl):
    th = theta(d_in=1152, d_out=1152, r=32)
    arr = (ctypes.POINTER(wl.Theta) * 1)(ctypes.pointer(th))
    lin = [wl.lib.wl_workspace_bytes(0, arr, 1, T) for T in (0, 1, 8, 64, 2048)]
    assert all(s > 0 and s % 256 == 0 for s in lin)
    # The MLP keeps h = [T][d_ff] bf16 in the workspace.
    g, u = theta(d_in=1152, d_out=6912, r=32), theta(W0=A + 0x100000, d_in=1152, d_out=6912, r=32)
    d = theta(W0=A + 0x200000, d_in=6912, d_out=1152, r=32)
    mlp_arr = (ctypes.POINTER(wl.Theta) * 3)(ctypes.pointer(g), ctypes.pointer(u), ctypes.pointer(d))
    mlp = [wl.lib.wl_workspace_bytes(2, mlp_arr, 3, T) for T in (1, 64, 2048)]
    assert mlp == sorted(mlp) and mlp[-1] >= 2048 * 6912 * 2
    assert wl.lib.wl_workspace_bytes(0, arr, 2, 1) == 0      # wrong count
    assert wl.lib.wl_workspace_bytes(7, arr, 1, 1) == 0      # unknown op
    assert wl.lib.wl_workspace_bytes(0, arr, 1, -1) == 0
    bad = theta(d_in=12)
    arr_bad = (ctypes.POINTER(wl.Theta) * 1)(ctypes.pointer(bad))
    assert wl.lib.wl_workspace_bytes(0, arr_bad, 1, 1) == 0


def test_output_overlap_is_rejected(wl):
    th = theta()
    # y on top of x
    assert call_linear(wl, th, x=D, y=D) == 1
    # y inside W0 (W0 spans 32*64*2 bytes from A)
    assert call_linear(wl, th, y=A + 256) == 1
    # y inside the workspace
    assert call_linear(wl, th, y=D + 0x2000000 + 4096) == 1
    assert b"overlap" in wl.lib.wl_last_error()


def test_qkv_requires_shared_d_in(wl):
    q, k = theta(d_in=64), theta(W0=A + 0x100000, d_in=64)
    v = theta(W0=A + 0x200000, d_in=128)
    rc = wl.lib.wl_qkv_fused(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), D, D + 0x1000000, 1,
                             D + 0x2000000, 1 << 30, None)
    assert rc == 1 and b"d_in" in wl.lib.wl_last_error()


def test_mlp_shape_checks(wl):
    gate = theta(W0=A, d_in=64, d_out=128)
    up = theta(W0=A + 0x100000, d_in=64, d_out=128)
    down_bad = theta(W0=A + 0x200000, d_in=64, d_out=64)
    rc = wl.lib.wl_mlp_fused(ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down_bad), D, D + 0x1000000,
                             1, D + 0x2000000, 1 << 30, None)
    assert rc == 1 and b"MLP" in wl.lib.wl_last_error()
    up_bad = theta(W0=A + 0x100000, d_in=64, d_out=120)
    down = theta(W0=A + 0x200000, d_in=128, d_out=64)
    rc = wl.lib.wl_mlp_fused(ctypes.byref(gate), ctypes.byref(up_bad), ctypes.byref(down), D, D + 0x1000000,
                             1, D + 0x2000000, 1 << 30, None)
    assert rc == 1


def test_weff_checks(wl):
    th = theta()
    assert wl.lib.wl_materialize_weff(ctypes.byref(th), None, None) == 1
    assert wl.lib.wl_materialize_weff(ctypes.byref(th), D + 2, None) == 1
    assert wl.lib.wl_materialize_weff(ctypes.byref(th), A, None) == 1     # on top of W0
    assert wl.lib.wl_materialize_weff(ctypes.byref(theta(r=99)), D, None) == 2


def weff_batch(wl, ths, outs):
    P = ctypes.POINTER(wl.Theta)
    arr = (P * len(ths))(*[ctypes.pointer(t) for t in ths])
    ptrs = (ctypes.c_void_p * len(outs))(*outs)
    return wl.lib.wl_materialize_weff_batch(arr, ptrs, len(ths), None)


def test_weff_batch_checks(wl):
    # Every case fails validation (or is the n = 0 no-op) before any launch.
    assert wl.lib.wl_materialize_weff_batch(None, None, 0, None) == 0
    assert wl.lib.wl_materialize_weff_batch(None, None, -1, None) == 1
    assert wl.lib.wl_materialize_weff_batch(None, None, 2, None) == 1
    t0, t1 = theta(), theta(W0=A + 0x100000, U=B + 0x100000, V=C + 0x100000)
    assert weff_batch(wl, [t0, theta(d_in=60)], [D, D + 0x100000]) == 1      # a bad second theta
    assert weff_batch(wl, [t0, theta(r=99)], [D, D + 0x100000]) == 2
    assert weff_batch(wl, [t0, t1], [D, None]) == 1
    assert weff_batch(wl, [t0, t1], [D, D + 0x100002]) == 1                   # misaligned
    assert weff_batch(wl, [t0, t1], [D, A + 0x100000]) == 1                   # on theta 1's W0
    assert weff_batch(wl, [t0, t1], [B + 0x100000, D]) == 1                   # output 0 on theta 1's U
    assert weff_batch(wl, [t0, t1], [D, D + 0x800]) == 1                      # the outputs overlap
    assert b"overlap" in wl.lib.wl_last_error()
    t1.dtype = 1
    assert weff_batch(wl, [t0, t1], [D, D + 0x100000]) == 1                   # two dtypes


def test_regime_switch(wl):
    prev = wl.set_regime(2)
    try:
        assert wl.set_regime(5) == 2
        assert wl.set_regime(6) == 5
        assert wl.set_regime(1) == 6
        with pytest.raises(ValueError):
            wl.set_regime(7)
    finally:
        wl.set_regime(prev)


def test_spin_limit_switch(wl):
    prev = wl.set_spin_limit(0)
    try:
        assert prev == 4096
        assert wl.set_spin_limit(7) == 0
        with pytest.raises(ValueError):
            wl.set_spin_limit(-1)
        assert wl.set_spin_limit(7) == 7
    finally:
        wl.set_spin_limit(prev)


def test_workspace_starts_with_the_sync_area(wl):
    # Every projection workspace holds the sync area before anything else.
    for d_in, d_out, r in ((1152, 1152, 32), (64, 8, 0)):
        th = theta(d_in=d_in, d_out=d_out, r=r)
        arr = (ctypes.POINTER(wl.Theta) * 1)(ctypes.pointer(th))
        assert wl.lib.wl_workspace_bytes(0, arr, 1, 1) >= wl.SYNC_BYTES + 256
    assert wl.SYNC_BYTES == wl.lib.wl_sync_bytes() == 9764864
    text = open(HEADER).read()
    assert re.search(r"#define WL_SYNC_BYTES 9764864\b", text)
    assert re.search(rf"#define WL_STATIC_SCRATCH_BYTES {wl.STATIC_SCRATCH_BYTES}\b", text)
    assert re.search(r"#define WL_ABI_VERSION 6\b", text)


def test_workspace_init_checks(wl):
    # validation only: every call below fails before anything is enqueued
    need = wl.SYNC_BYTES
    assert wl.lib.wl_workspace_init(None, need, None) == 1
    assert wl.lib.wl_workspace_init(A + 0x10, need, None) == 1          # misaligned
    assert wl.lib.wl_workspace_init(A, need - 1, None) == 4              # below the sync area
    assert b"sync area" in wl.lib.wl_last_error()


def test_library_resolves_its_own_symbols(wl):
    # A kernel whose host stub was not emitted shows up as an undefined symbol
    # of the library's own namespace; loading would then fail on the GPU machine.
    out = subprocess.run(["nm", "-u", "-C", wl.LIBRARY], capture_output=True, text=True, check=True).stdout
    own = [line for line in out.splitlines() if "wl::" in line]
    assert not own, f"unresolved library symbols: {own}"


def bundle(wl, thetas):
    arr = (ctypes.POINTER(wl.Theta) * len(thetas))(*[ctypes.pointer(t) for t in thetas])
    b, d = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = wl.lib.wl_bundle_size(arr, len(thetas), ctypes.byref(b), ctypes.byref(d))
    return st, b.value, d.value


# Gemma-3-1B-shaped families (d_in, d_out): q, k, v, o, gate, up, down.
FAMILIES = ((1152, 1024), (1152, 256), (1152, 256), (1024, 1152), (1152, 6912), (1152, 6912), (6912, 1152))


def layer_thetas(wl, r, n_layers, shared):
    # Fake, distinct 256-byte aligned W0 addresses; with `shared` every layer uses
    # the same W0 per family (one band of n_layers layers).
    out = []
    for layer in range(n_layers):
        for f, (d_in, d_out) in enumerate(FAMILIES):
            w0 = A + 0x100 * (f if shared else layer * len(FAMILIES) + f)
            out.append(wl.Theta(w0, B, C, D, d_in, d_out, r))
    return out


@pytest.mark.parametrize("r,ratio", [(4, 0.0445), (16, 0.0585), (32, 0.0772)])
def test_bundle_ratio_of_shared_w0_layers(wl, r, ratio):
    # 26 layers sharing one W0 per family against 26 dense layers: the ratios
    # derived for the batched-decode shapes (theta bundle over original weights).
    st, b, d = bundle(wl, layer_thetas(wl, r, 26, shared=True))
    assert st == 0
    assert d == 26 * sum(2 * i * o for i, o in FAMILIES)
    assert round(b / d, 4) == ratio


def test_bundle_of_own_w0_layers_exceeds_dense(wl):
    # One W0 per layer: the bundle is the dense size plus s, U and V (1.006 to 1.039).
    for r, lo, hi in ((4, 1.005, 1.007), (32, 1.038, 1.040)):
        st, b, d = bundle(wl, layer_thetas(wl, r, 26, shared=False))
        assert st == 0 and lo < b / d < hi


def test_bundle_checks(wl):
    t = [wl.Theta(A, None, B, C, 64, 32, 4), wl.Theta(A, None, B, C, 64, 48, 4)]
    assert bundle(wl, t)[0] == 1                      # shared W0 with another shape
    assert bundle(wl, [wl.Theta(A, None, B, C, 60, 32, 4)])[0] == 1
    st, b, d = bundle(wl, [wl.Theta(A, None, B, C, 64, 32, 0)])
    assert (st, b, d) == (0, 2 * 64 * 32, 2 * 64 * 32)   # r = 0, no s: the bundle is W0 itself


# -- the fp32 variant: host checks ------------------------------------------------------------

F32 = 1


def test_dtype_is_checked(wl):
    bad = theta()
    bad.dtype = 2
    assert call_linear(wl, bad) == 2 and b"dtype" in wl.lib.wl_last_error()
    arr = (ctypes.POINTER(wl.Theta) * 1)(ctypes.pointer(bad))
    assert wl.lib.wl_workspace_bytes(0, arr, 1, 1) == 0


def test_fused_calls_need_one_dtype(wl):
    q, k = theta(d_in=64), theta(W0=A + 0x100000, d_in=64)
    v = theta(W0=A + 0x200000, d_in=64)
    k.dtype = F32
    rc = wl.lib.wl_qkv_fused(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), D, D + 0x1000000, 1,
                             D + 0x2000000, 1 << 30, None)
    assert rc == 1 and b"dtype" in wl.lib.wl_last_error()
    gate, up = theta(W0=A, d_in=64, d_out=128), theta(W0=A + 0x100000, d_in=64, d_out=128)
    down = theta(W0=A + 0x200000, d_in=128, d_out=64)
    down.dtype = F32
    rc = wl.lib.wl_mlp_fused(ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down), D, D + 0x1000000,
                             1, D + 0x2000000, 1 << 30, None)
    assert rc == 1 and b"dtype" in wl.lib.wl_last_error()


def test_f32_sizes(wl):
    # Overlap checks count 4-byte elements: W0 of 32 x 64 fp32 spans 8192 bytes from A.
    th = theta()
    th.dtype = F32
    assert call_linear(wl, th, y=A + 5120) == 1 and b"overlap" in wl.lib.wl_last_error()
    # The fp32 MLP keeps h = [T][d_ff] fp32 in the workspace.
    g, u = theta(d_in=1152, d_out=6912, r=32), theta(W0=A + 0x100000, d_in=1152, d_out=6912, r=32)
    d = theta(W0=A + 0x200000, d_in=6912, d_out=1152, r=32)
    for t_ in (g, u, d):
        t_.dtype = F32
    mlp_arr = (ctypes.POINTER(wl.Theta) * 3)(ctypes.pointer(g), ctypes.pointer(u), ctypes.pointer(d))
    sizes = [wl.lib.wl_workspace_bytes(2, mlp_arr, 3, T) for T in (1, 8, 2048)]
    assert sizes == sorted(sizes) and sizes[-1] >= 2048 * 6912 * 4 and all(s % 256 == 0 for s in sizes)
    # Bundle sizes count 4 bytes per fp32 element; a W0 shared across dtypes is an error.
    st, b, dn = bundle(wl, [wl.Theta(A, None, B, C, 64, 32, 0, F32)])
    assert (st, b, dn) == (0, 4 * 64 * 32, 4 * 64 * 32)
    st, b, dn = bundle(wl, [wl.Theta(A, D, B, C, 64, 32, 2, F32)])
    assert (st, b, dn) == (0, 4 * 64 * 32 + 4 * 32 + 4 * 2 * (32 + 64), 4 * 64 * 32)
    assert bundle(wl, [wl.Theta(A, None, B, C, 64, 32, 0, F32), wl.Theta(A, None, B, C, 64, 32, 0, 0)])[0] == 1


def test_rel_frob_checks(wl):
    f = wl.lib.wl_relative_frobenius_error
    need = wl.lib.wl_rel_frob_workspace_bytes(1 << 20)
    assert need >= 16 and need % 256 == 0
    assert wl.lib.wl_rel_frob_workspace_bytes(0) == 0
    assert f(None, B, 64, C, D, need, None) == 1
    assert f(A + 2, B, 64, C, D, need, None) == 1                # misaligned W
    assert f(A, B, 0, C, D, need, None) == 1                     # empty
    assert f(A, B, 64, C + 4, D, need, None) == 1                # misaligned result
    assert f(A, B, 64, C, D, 0, None) == 4                       # workspace too small
    assert f(A, B, 64, A + 8, D, need, None) == 1                # result on top of W


def _calls(wl, specs):
    """ctypes call array from (op, [theta structs], x, y, T) tuples; keeps the structs alive."""
    arr = (wl.Call * len(specs))()
    keep = []
    for i, (op, ths, x, y, T) in enumerate(specs):
        keep.append(ths)
        arr[i].op = op
        for j, t in enumerate(ths):
            arr[i].th[j] = ctypes.pointer(t)
        arr[i].x, arr[i].y, arr[i].T = x, y, T
    return arr, keep


def _create(wl, arr, n, flags=0, ws=D + 0x2000000, ws_bytes=1 << 30):
    h = ctypes.c_void_p()
    st = wl.lib.wl_step_create(arr, n, flags, ws, ws_bytes, ctypes.byref(h))
    return st, h


def test_step_validation_before_any_launch(wl):
    lin = theta(d_in=64, d_out=32)
    arr, keep = _calls(wl, [(wl.OP_LINEAR, [lin], D, D + 0x100000, 2)])
    need = wl.lib.wl_step_workspace_bytes(arr, 1)
    assert need >= wl.SYNC_BYTES
    assert wl.lib.wl_step_workspace_bytes(arr, 0) == 0
    assert _create(wl, arr, 0)[0] == wl.WL_ERR_INVALID_ARG                 # no calls
    assert wl.lib.wl_step_create(arr, 1, 0, D + 0x2000000, 1 << 30, None) == wl.WL_ERR_INVALID_ARG
    assert _create(wl, arr, 1, flags=4)[0] == wl.WL_ERR_INVALID_ARG        # unknown flag
    assert _create(wl, arr, 1, ws_bytes=need - 256)[0] == wl.WL_ERR_WORKSPACE
    assert _create(wl, arr, 1, ws=D + 0x2000000 + 8)[0] == wl.WL_ERR_INVALID_ARG   # misaligned
    bad, keep2 = _calls(wl, [(7, [lin], D, D + 0x100000, 2)])
    st, h = _create(wl, bad, 1)
    assert st == wl.WL_ERR_INVALID_ARG and h.value is None
    assert b"call 0" in wl.lib.wl_last_error()
    nul = (wl.Call * 1)()
    nul[0].op = wl.OP_MLP
    assert _create(wl, nul, 1)[0] == wl.WL_ERR_INVALID_ARG                  # NULL thetas
    assert wl.lib.wl_step_destroy(None) == 0
    assert wl.lib.wl_step_launch(None, None) == wl.WL_ERR_INVALID_ARG


def test_step_grouping_needs_independent_calls(wl):
    a, b = theta(W0=A, d_in=64, d_out=64), theta(W0=A, d_in=64, d_out=64)
    y1, y2 = D + 0x100000, D + 0x200000
    # call 1 reads call 0's output: fine in given order, refused when regrouping
    arr, keep = _calls(wl, [(wl.OP_LINEAR, [a], D, y1, 2), (wl.OP_LINEAR, [b], y1, y2, 2)])
    st, h = _create(wl, arr, 2, flags=wl.STEP_GROUP_SHARED_W0)
    assert st == wl.WL_ERR_INVALID_ARG and b"reads the output" in wl.lib.wl_last_error()
    # two calls writing overlapping outputs
    arr, keep = _calls(wl, [(wl.OP_LINEAR, [a], D, y1, 2), (wl.OP_LINEAR, [b], D, y1 + 64, 2)])
    st, h = _create(wl, arr, 2, flags=wl.STEP_GROUP_SHARED_W0)
    assert st == wl.WL_ERR_INVALID_ARG and b"overlapping outputs" in wl.lib.wl_last_error()
