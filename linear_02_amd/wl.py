"""Python binding of libwl (the C ABI in include/wl.h).

Argument marshalling only: every function here checks tensor dtypes, shapes
and devices, passes raw device pointers and the current HIP stream to the
library, and returns the output tensor. All arithmetic runs in the library's
HIP kernels; there is no fallback of any kind. If libwl.so is missing the
import fails loudly (build it with ``python -m linear_02_amd.build``).

A theta is a dict with device tensors ``W0`` ([d_out][d_in]), ``s`` (fp32
[d_out] or None), ``U`` ([d_out][r]), ``V`` ([d_in][r]) and the ints ``d_in``,
``d_out``, ``r``, as drawn by ``linear_02_amd.inputs.theta`` and moved with
:func:`theta_to`. W0, U, V, x and the outputs are all bf16 or all fp32 (the
dtype of W0 picks the variant).
"""
from __future__ import annotations

import ctypes
import os

import torch

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwl.so")

OP_LINEAR, OP_QKV, OP_MLP = 0, 1, 2
ABI_VERSION = 6
# The first SYNC_BYTES of a projection workspace are the library's sync area:
# cleared by wl_workspace_init (new_workspace does it) before first use, then
# written only by the library's calls.
SYNC_BYTES = 9764864
# Bytes of the static workspace wl_linear_static uses on each device.
STATIC_SCRATCH_BYTES = 33554432
_FALLBACK_WORD = 511   # int64 word of the sync area counting decode workgroups that stopped waiting
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "HIP error", 4: "workspace too small"}
WL_OK, WL_ERR_INVALID_ARG, WL_ERR_UNSUPPORTED, WL_ERR_HIP, WL_ERR_WORKSPACE = 0, 1, 2, 3, 4


class WlError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


DTYPE_BF16, DTYPE_F32 = 0, 1
_CODES = {torch.bfloat16: DTYPE_BF16, torch.float32: DTYPE_F32}


class Theta(ctypes.Structure):
    _fields_ = [("W0", ctypes.c_void_p), ("s", ctypes.c_void_p), ("U", ctypes.c_void_p),
                ("V", ctypes.c_void_p), ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32),
                ("r", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Call(ctypes.Structure):
    _fields_ = [("op", ctypes.c_int32), ("th", ctypes.POINTER(Theta) * 3), ("x", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("T", ctypes.c_int32)]


STEP_GROUP_SHARED_W0 = 1


def _load(path: str = LIBRARY) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m linear_02_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(Theta)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.wl_workspace_bytes.argtypes = [i32, ctypes.POINTER(P), i32, i32]
    lib.wl_workspace_bytes.restype = sz
    lib.wl_linear.argtypes = [P, vp, vp, i32, vp, sz, vp]
    lib.wl_linear_static.argtypes = [P, vp, vp, i32, vp]
    lib.wl_qkv_fused.argtypes = [P, P, P, vp, vp, i32, vp, sz, vp]
    lib.wl_mlp_fused.argtypes = [P, P, P, vp, vp, i32, vp, sz, vp]
    lib.wl_materialize_weff.argtypes = [P, vp, vp]
    lib.wl_materialize_weff_batch.argtypes = [ctypes.POINTER(P), ctypes.POINTER(vp), i32, vp]
    lib.wl_materialize_weff_batch.restype = ctypes.c_int
    for name in ("wl_linear", "wl_linear_static", "wl_qkv_fused", "wl_mlp_fused", "wl_materialize_weff"):
        getattr(lib, name).restype = ctypes.c_int
    lib.wl_set_regime.argtypes = [i32]
    lib.wl_set_regime.restype = i32
    lib.wl_set_spin_limit.argtypes = [i32]
    lib.wl_set_spin_limit.restype = i32
    lib.wl_status_str.argtypes = [ctypes.c_int]
    lib.wl_status_str.restype = ctypes.c_char_p
    lib.wl_last_error.argtypes = []
    lib.wl_last_error.restype = ctypes.c_char_p
    lib.wl_abi_version.argtypes = []
    lib.wl_abi_version.restype = i32
    lib.wl_bundle_size.argtypes = [ctypes.POINTER(P), i32, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.wl_bundle_size.restype = ctypes.c_int
    lib.wl_rel_frob_workspace_bytes.argtypes = [ctypes.c_int64]
    lib.wl_rel_frob_workspace_bytes.restype = sz
    lib.wl_relative_frobenius_error.argtypes = [vp, vp, ctypes.c_int64, vp, vp, sz, vp]
    lib.wl_relative_frobenius_error.restype = ctypes.c_int
    lib.wl_step_workspace_bytes.argtypes = [ctypes.POINTER(Call), i32]
    lib.wl_step_workspace_bytes.restype = sz
    lib.wl_step_create.argtypes = [ctypes.POINTER(Call), i32, i32, vp, sz, ctypes.POINTER(vp)]
    lib.wl_step_create.restype = ctypes.c_int
    lib.wl_step_launch.argtypes = [vp, vp]
    lib.wl_step_launch.restype = ctypes.c_int
    lib.wl_step_destroy.argtypes = [vp]
    lib.wl_step_destroy.restype = ctypes.c_int
    lib.wl_workspace_init.argtypes = [vp, sz, vp]
    lib.wl_workspace_init.restype = ctypes.c_int
    lib.wl_sync_bytes.argtypes = []
    lib.wl_sync_bytes.restype = sz
    if lib.wl_abi_version() != ABI_VERSION or lib.wl_sync_bytes() != SYNC_BYTES:
        raise ImportError(f"{path}: ABI version {lib.wl_abi_version()} / sync area {lib.wl_sync_bytes()} bytes, "
                          f"this binding expects {ABI_VERSION} / {SYNC_BYTES}; rebuild the library")
    return lib


lib = _load()


def _check(status: int) -> None:
    if status != 0:
        raise WlError(status, lib.wl_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def theta_to(th: dict, device) -> dict:
    """Copy a theta's tensors to ``device`` (contiguous); ints are kept."""
    out = dict(th)
    for key in ("W0", "s", "U", "V"):
        if th.get(key) is not None:
            out[key] = th[key].to(device).contiguous()
    return out


def make_theta(th: dict) -> Theta:
    """The C struct of a theta dict (device tensors). The dict keeps them alive."""
    W0, s, U, V = th["W0"], th.get("s"), th.get("U"), th.get("V")
    d_in, d_out, r = int(th["d_in"]), int(th["d_out"]), int(th["r"])
    if W0.dtype not in _CODES or not W0.is_contiguous() or tuple(W0.shape) != (d_out, d_in):
        raise ValueError("W0 must be a contiguous bf16 or fp32 [d_out][d_in] tensor")
    if s is not None and (s.dtype != torch.float32 or not s.is_contiguous() or s.numel() != d_out):
        raise ValueError("s must be a contiguous fp32 [d_out] tensor or None")
    if r > 0:
        for name, t, rows in (("U", U, d_out), ("V", V, d_in)):
            if t is None or t.dtype != W0.dtype or not t.is_contiguous() or tuple(t.shape) != (rows, r):
                raise ValueError(f"{name} must be a contiguous [{rows}][{r}] tensor of W0's dtype")
    return Theta(_ptr(W0), _ptr(s), _ptr(U) if r > 0 else None, _ptr(V) if r > 0 else None, d_in, d_out, r,
                 _CODES[W0.dtype])


def workspace_bytes(op: int, thetas: list, T: int) -> int:
    structs = [make_theta(t) for t in thetas]
    arr = (ctypes.POINTER(Theta) * len(structs))(*[ctypes.pointer(s) for s in structs])
    return int(lib.wl_workspace_bytes(op, arr, len(structs), T))


def workspace_init(ws: torch.Tensor) -> None:
    """Clear the sync area of a projection workspace (wl_workspace_init, on the
    current stream)."""
    _check(lib.wl_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(ws.device)))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A projection workspace of at least nbytes (and at least the sync area),
    prepared by wl_workspace_init."""
    device = torch.device(device)
    ws = torch.empty(max(int(nbytes), SYNC_BYTES), dtype=torch.uint8, device=device)
    workspace_init(ws)
    return ws


class Workspace:
    """A device workspace per (device, stream) that grows on demand, prepared by
    wl_workspace_init when allocated.

    Calls on one stream run in order, so they can share one workspace."""

    def __init__(self):
        self._bufs: dict = {}

    def get(self, device: torch.device, nbytes: int) -> torch.Tensor | None:
        if nbytes == 0:
            return None
        key = (device.index, torch.cuda.current_stream(device).cuda_stream)
        buf = self._bufs.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = new_workspace(max(nbytes, 1 << 20), device)
            self._bufs[key] = buf
        return buf


WORKSPACE = Workspace()


def _io(x: torch.Tensor, d_in: int, dtype: torch.dtype) -> int:
    if x.dtype != dtype or not x.is_contiguous() or x.dim() != 2 or x.shape[1] != d_in:
        raise ValueError(f"x must be a contiguous {dtype} [T][{d_in}] tensor")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    return x.shape[0]


def wl_linear(th: dict, x: torch.Tensor, y: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """y = s (.) (W0 x) + U (V^T x), [T][d_out] of W0's dtype."""
    T = _io(x, int(th["d_in"]), th["W0"].dtype)
    st = make_theta(th)
    if y is None:
        y = torch.empty(T, int(th["d_out"]), dtype=th["W0"].dtype, device=x.device)
    need = workspace_bytes(OP_LINEAR, [th], T)
    ws = ws if ws is not None else WORKSPACE.get(x.device, need)
    _check(lib.wl_linear(ctypes.byref(st), _ptr(x), _ptr(y), T, _ptr(ws),
                         0 if ws is None else ws.numel() * ws.element_size(), _stream(x.device)))
    return y


def wl_linear_static(th: dict, x: torch.Tensor, y: torch.Tensor | None = None):
    """wl_linear with the library's static workspace (no workspace argument;
    the C call allocates no device memory). y is allocated here when not given."""
    T = _io(x, int(th["d_in"]), th["W0"].dtype)
    st = make_theta(th)
    if y is None:
        y = torch.empty(T, int(th["d_out"]), dtype=th["W0"].dtype, device=x.device)
    _check(lib.wl_linear_static(ctypes.byref(st), _ptr(x), _ptr(y), T, _stream(x.device)))
    return y


def wl_qkv_fused(q: dict, k: dict, v: dict, x: torch.Tensor, y: torch.Tensor | None = None,
                 ws: torch.Tensor | None = None):
    """Q | K | V side by side, [T][dq + dk + dv] of the thetas' dtype."""
    T = _io(x, int(q["d_in"]), q["W0"].dtype)
    sq, sk, sv = make_theta(q), make_theta(k), make_theta(v)
    width = int(q["d_out"]) + int(k["d_out"]) + int(v["d_out"])
    if y is None:
        y = torch.empty(T, width, dtype=q["W0"].dtype, device=x.device)
    need = workspace_bytes(OP_QKV, [q, k, v], T)
    ws = ws if ws is not None else WORKSPACE.get(x.device, need)
    _check(lib.wl_qkv_fused(ctypes.byref(sq), ctypes.byref(sk), ctypes.byref(sv), _ptr(x), _ptr(y), T,
                            _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(x.device)))
    return y


def wl_mlp_fused(gate: dict, up: dict, down: dict, x: torch.Tensor, y: torch.Tensor | None = None,
                 ws: torch.Tensor | None = None):
    """down(round(gelu_tanh(gate x) * up x)), [T][down.d_out] of the thetas' dtype."""
    T = _io(x, int(gate["d_in"]), gate["W0"].dtype)
    sg, su, sd = make_theta(gate), make_theta(up), make_theta(down)
    if y is None:
        y = torch.empty(T, int(down["d_out"]), dtype=gate["W0"].dtype, device=x.device)
    need = workspace_bytes(OP_MLP, [gate, up, down], T)
    ws = ws if ws is not None else WORKSPACE.get(x.device, need)
    _check(lib.wl_mlp_fused(ctypes.byref(sg), ctypes.byref(su), ctypes.byref(sd), _ptr(x), _ptr(y), T,
                            _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(x.device)))
    return y


def wl_materialize_weff(th: dict, W_eff: torch.Tensor | None = None):
    """W_eff = round(s (.) W0 + U V^T), [d_out][d_in] of W0's dtype."""
    st = make_theta(th)
    dev = th["W0"].device
    if W_eff is None:
        W_eff = torch.empty(int(th["d_out"]), int(th["d_in"]), dtype=th["W0"].dtype, device=dev)
    _check(lib.wl_materialize_weff(ctypes.byref(st), _ptr(W_eff), _stream(dev)))
    return W_eff


def wl_materialize_weff_batch(thetas: list, W_effs: list | None = None) -> list:
    """wl_materialize_weff for every theta in one launch per eight; returns the
    W_eff tensors (allocated when W_effs is None)."""
    if not thetas:
        return []
    dev = thetas[0]["W0"].device
    if W_effs is None:
        W_effs = [torch.empty(int(t["d_out"]), int(t["d_in"]), dtype=t["W0"].dtype, device=dev) for t in thetas]
    structs = [make_theta(t) for t in thetas]
    arr = (ctypes.POINTER(Theta) * len(structs))(*[ctypes.pointer(st) for st in structs])
    outs = (ctypes.c_void_p * len(W_effs))(*[_ptr(w) for w in W_effs])
    _check(lib.wl_materialize_weff_batch(arr, outs, len(structs), _stream(dev)))
    return W_effs


def bundle_size(thetas: list) -> tuple:
    """(bundle bytes, dense bytes) of a set of thetas: each distinct W0 counted once,
    s, U and V per theta, against the dense weights (of the thetas' dtype) they stand for."""
    structs = [make_theta(t) for t in thetas]
    arr = (ctypes.POINTER(Theta) * len(structs))(*[ctypes.pointer(st) for st in structs])
    b, d = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib.wl_bundle_size(arr, len(structs), ctypes.byref(b), ctypes.byref(d)))
    return int(b.value), int(d.value)


def relative_frobenius_error(W: torch.Tensor, R: torch.Tensor) -> float:
    """||W - R||_F / ||W||_F of two bf16 device tensors of equal size (waits for the
    result)."""
    for name, t in (("W", W), ("R", R)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous bf16 device tensor")
    if W.numel() != R.numel():
        raise ValueError("W and R must have the same number of elements")
    n = W.numel()
    out = torch.empty(1, dtype=torch.float64, device=W.device)
    ws = torch.empty(max(int(lib.wl_rel_frob_workspace_bytes(n)), 256), dtype=torch.uint8, device=W.device)
    _check(lib.wl_relative_frobenius_error(_ptr(W), _ptr(R), n, _ptr(out), _ptr(ws),
                                            ws.numel(), _stream(W.device)))
    return float(out.item())


REGIME_AUTO, REGIME_GEMV, REGIME_MFMA, REGIME_GEMV_TWO_LAUNCH, REGIME_SKINNY, REGIME_GEMV_MLP_SPLIT = 0, 1, 2, 3, 4, 5


def set_regime(regime: int) -> int:
    """0 auto, 1 decode kernels (the MLP in one launch where it applies), 2
    matrix-core GEMM, 3 decode GEMV always after a separate V^T x launch, 4
    few-token split path, 5 as 1 with the MLP as two launches, 6 as 2 with
    V^T x always in a launch of its own and the rank term in the GEMM epilogue;
    returns the previous setting (wl_testing.h)."""
    prev = int(lib.wl_set_regime(regime))
    if prev < 0:
        raise ValueError(f"regime {regime} is not one of 0 to 6")
    return prev


def set_spin_limit(polls: int) -> int:
    """Times a decode workgroup reads each group of in-launch V^T x words before
    it computes V^T x itself (0: at once); returns the previous setting."""
    prev = int(lib.wl_set_spin_limit(polls))
    if prev < 0:
        raise ValueError(f"spin limit {polls} is negative")
    return prev


def fallback_count(ws: torch.Tensor) -> int:
    """Decode workgroups, over all calls on workspace ``ws`` so far, whose wait
    for the in-launch V^T x ran out (a counter in the sync area); waits for the
    device."""
    w = _FALLBACK_WORD * 8
    return int(ws[w:w + 8].view(torch.int64).item())


def abi_version() -> int:
    return int(lib.wl_abi_version())


class Step:
    """A decode step: a fixed list of calls that the library records once into a
    HIP graph (wl_step_create) and launches with one call.

    calls: (op, thetas, x, y) tuples, op one of OP_LINEAR (one theta), OP_QKV
    (Q, K, V), OP_MLP (gate, up, down); device tensors, which must stay alive
    while the step exists (the step keeps references). group_shared_w0 launches
    calls that share their first theta's W0 back to back (independent calls
    only)."""

    def __init__(self, calls, ws: torch.Tensor | None = None, group_shared_w0: bool = False):
        n = len(calls)
        arr = (Call * n)()
        self._keep = []
        device = None
        for i, (op, thetas, x, y) in enumerate(calls):
            if len(thetas) != (1 if op == OP_LINEAR else 3):
                raise ValueError(f"call {i}: {len(thetas)} thetas for op {op}")
            T = _io(x, int(thetas[0]["d_in"]), thetas[0]["W0"].dtype)
            structs = [make_theta(t) for t in thetas]
            self._keep += [structs, thetas, x, y]
            arr[i].op = op
            for j, st in enumerate(structs):
                arr[i].th[j] = ctypes.pointer(st)
            arr[i].x, arr[i].y, arr[i].T = _ptr(x), _ptr(y), T
            device = x.device
        need = int(lib.wl_step_workspace_bytes(arr, n))
        if need == 0:
            raise ValueError("invalid calls for a step")
        self.ws = ws if ws is not None else new_workspace(need, device)
        self.device = device
        h = ctypes.c_void_p()
        _check(lib.wl_step_create(arr, n, STEP_GROUP_SHARED_W0 if group_shared_w0 else 0, _ptr(self.ws),
                                  self.ws.numel() * self.ws.element_size(), ctypes.byref(h)))
        self.handle = h

    def launch(self) -> None:
        _check(lib.wl_step_launch(self.handle, _stream(self.device)))

    def close(self) -> None:
        if getattr(self, "handle", None) is not None and self.handle.value:
            torch.cuda.current_stream(self.device).synchronize()
            lib.wl_step_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
