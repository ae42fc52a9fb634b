"""Seeded synthetic inputs for the reconstruct-and-project linear.

This module only draws numbers. It holds none of the method's arithmetic: no
product, sum, scale or activation of the projection is computed here. Both the
HIP path (through the tests and the benchmark) and the CPU oracle take their
inputs from these generators, so parity never depends on two RNGs agreeing.

A theta bundle is one projection's factors, named as on the "In-kernel
reconstruction" page (reconstruction equation and its per-element expansion):

  W0[o, i]  bf16, shape [d_out][d_in]   the shared block (shared per band of
                                        layers, "Serve and generate with
                                        weightless", introduction)
  s[o]      fp32, shape [d_out]         per-output-row scale
  U[o, k]   bf16, shape [d_out][r]      low-rank up factor
  V[i, k]   bf16, shape [d_in][r]       low-rank down factor

Activations x[t, i] are bf16 [T][d_in]. Values are drawn in fp32 from a normal
distribution (the second argument is the standard deviation) and rounded to
bf16 with round-to-nearest-even by torch's dtype conversion; s stays fp32.
With ``dtype=torch.float32`` (the fp32 variant of every operation) the same
draws are kept in fp32 unrounded.

The pages print no checkpoint values, so these draws stand in for the Gemma
checkpoints their measurements use.
"""
from __future__ import annotations

import torch

# Projection shapes of the two model families the pages serve.
# Gemma 3 1B: hidden 1152, 4 query heads x 256, one 256-wide KV head, MLP 6912.
GEMMA3_1B = dict(d_model=1152, q=1024, kv=256, ff=6912, layers=26)
# The large-model layer: hidden 5376, Q 8192, K/V 2048 each, MLP 21504.
LARGE_5376 = dict(d_model=5376, q=8192, kv=2048, ff=21504, layers=60)

FAMILIES = ("q", "k", "v", "o", "gate", "up", "down")


def family_shapes(dims: dict) -> dict:
    """(d_in, d_out) of every projection family of one decoder layer."""
    d, q, kv, ff = dims["d_model"], dims["q"], dims["kv"], dims["ff"]
    return {
        "q": (d, q), "k": (d, kv), "v": (d, kv), "o": (q, d),
        "gate": (d, ff), "up": (d, ff), "down": (ff, d),
    }


def _normal(gen: torch.Generator, shape, std: float, mean: float = 0.0) -> torch.Tensor:
    t = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t


def theta(gen: torch.Generator, d_in: int, d_out: int, r: int, *,
          w0_std: float = 0.02, uv_std: float = 0.01, s_std: float = 0.01,
          W0: torch.Tensor | None = None, dtype: torch.dtype = torch.bfloat16) -> dict:
    """Draw one theta bundle (CPU tensors). Draw order: W0 (unless given), s, U, V.
    W0, U and V are ``dtype`` (bf16 or fp32); s is fp32."""
    if W0 is None:
        W0 = _normal(gen, (d_out, d_in), w0_std).to(dtype)
    else:
        assert tuple(W0.shape) == (d_out, d_in) and W0.dtype == dtype
    s = _normal(gen, (d_out,), s_std, mean=1.0)
    U = _normal(gen, (d_out, r), uv_std).to(dtype)
    V = _normal(gen, (d_in, r), uv_std).to(dtype)
    return dict(W0=W0, s=s, U=U, V=V, d_in=d_in, d_out=d_out, r=r)


def activations(gen: torch.Generator, T: int, d: int, std: float = 1.0,
                dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """x ~ N(0, std) as ``dtype`` (bf16: rounded), shape [T][d]."""
    return _normal(gen, (T, d), std).to(dtype)


def layer(gen: torch.Generator, dims: dict, r: int, *, w0_std: float = 0.02,
          shared_W0: dict | None = None, dtype: torch.dtype = torch.bfloat16) -> dict:
    """One decoder layer's seven theta bundles, drawn in the fixed family order.

    ``shared_W0`` maps family -> an already-drawn W0 (band sharing: one W0 per
    band of layers); such a W0 is reused and not drawn again.
    """
    shapes = family_shapes(dims)
    out = {}
    for fam in FAMILIES:
        d_in, d_out = shapes[fam]
        w = None if shared_W0 is None else shared_W0.get(fam)
        out[fam] = theta(gen, d_in, d_out, r, w0_std=w0_std, W0=w, dtype=dtype)
    return out


def layer_inputs(gen: torch.Generator, dims: dict, T: int, dtype: torch.dtype = torch.bfloat16) -> dict:
    """The three distinct projection inputs of a layer: attention input (feeds
    Q/K/V), attention output (feeds O) and MLP input (feeds gate/up)."""
    return dict(
        x_attn=activations(gen, T, dims["d_model"], dtype=dtype),
        x_o=activations(gen, T, dims["q"], dtype=dtype),
        x_mlp=activations(gen, T, dims["d_model"], dtype=dtype),
    )


def layers(gen: torch.Generator, dims: dict, r: int, n_layers: int, G: int, *,
           w0_std: float = 0.02, dtype: torch.dtype = torch.bfloat16) -> list:
    """``n_layers`` layers with ``G`` distinct W0 blocks per family: layer l uses
    block l // ceil(n_layers / G) (bands of consecutive layers). G == n_layers is
    the passthrough point (own W0 per layer); G == 1 shares one W0 everywhere."""
    assert 1 <= G <= n_layers
    band = -(-n_layers // G)
    out, bands = [], {}
    for l in range(n_layers):
        b = l // band
        lay = layer(gen, dims, r, w0_std=w0_std, shared_W0=bands.get(b), dtype=dtype)
        bands.setdefault(b, {f: lay[f]["W0"] for f in FAMILIES})
        out.append(lay)
    return out


# Exactly representable inputs ---------------------------------------------------------
# Small integers (and halves / powers of two for s) are exact in bf16 and fp32, so every
# partial sum of a small problem is exact in any summation order. These serve the
# bit-exact parity cases.

def int_tensor(gen: torch.Generator, shape, lo: int, hi: int, dtype=torch.bfloat16,
               density: float = 1.0) -> torch.Tensor:
    """Uniform integers in [lo, hi]; with density < 1 the rest are zero."""
    v = torch.randint(lo, hi + 1, tuple(shape), generator=gen, dtype=torch.int64)
    if density < 1.0:
        keep = torch.rand(tuple(shape), generator=gen) < density
        v = v * keep
    return v.to(dtype)


def choice_tensor(gen: torch.Generator, shape, values, dtype=torch.float32) -> torch.Tensor:
    """Entries drawn uniformly from ``values``."""
    vals = torch.tensor(values, dtype=torch.float64)
    idx = torch.randint(0, len(values), tuple(shape), generator=gen)
    return vals[idx].to(dtype)


def sparse_pm1_rows(gen: torch.Generator, T: int, d: int, nnz: int) -> torch.Tensor:
    """bf16 [T][d] with exactly ``nnz`` entries of +-1 per row, the rest zero."""
    out = torch.zeros(T, d, dtype=torch.float32)
    for t in range(T):
        cols = torch.randperm(d, generator=gen)[:nnz]
        signs = torch.randint(0, 2, (nnz,), generator=gen).to(torch.float32) * 2 - 1
        out[t, cols] = signs
    return out.to(torch.bfloat16)
