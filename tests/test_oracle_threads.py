"""The oracle's values do not depend on its OpenMP thread count.

Each output element (and each V^T x entry, h entry and W_eff entry) is one
thread's sequential fp64 loop, so one thread and several give the same bits.
"""
from __future__ import annotations

import numpy as np
import torch

from linear_02_amd import inputs


def _all_ops(orc, g_seed: int):
    g = torch.Generator().manual_seed(g_seed)
    q, k, v = (inputs.theta(g, 136, d, r) for d, r in ((96, 8), (40, 3), (40, 0)))
    gate, up = inputs.theta(g, 136, 200, 5), inputs.theta(g, 136, 200, 0)
    down = inputs.theta(g, 200, 72, 16)
    x = inputs.activations(g, 7, 136)
    out = []
    out += list(orc.linear(q, x))
    out += list(orc.qkv(q, k, v, x))
    y, b, h = orc.mlp(gate, up, down, x)
    out += [y, b, h.astype(np.float64)]
    out += list(orc.weff(down))
    return out


def test_thread_count_does_not_change_values(orc):
    prev = orc.threads()
    try:
        orc.threads(1)
        one = _all_ops(orc, 31)
        orc.threads(max(prev, 4))
        assert orc.threads() == max(prev, 4)
        many = _all_ops(orc, 31)
    finally:
        orc.threads(prev)
    for a, b in zip(one, many):
        assert np.array_equal(a.view(np.uint64), b.view(np.uint64))
