"""The gate projections of the gated layer (oracle).  TEST INFRASTRUCTURE ONLY.

[SA-ja] ゲート付き SA と SWA の組み合わせ: the weights g_sa and g_swa come from independent sigmoid
projections of the layer input.  Reading (R21): g_path[b, i, h] = sigmoid(<x[b, i], w[:, j]> +
bias[j]), with column j = path * Hq + h of one projection matrix w [Hm, 2 Hq] (the SA gates'
columns first), in float64.

Pins (tests/test_oracle_gates.py): zero input gives sigmoid(bias); a one-hot input picks one row
of w; negating w and the bias reflects every gate g -> 1 - g.
"""

from __future__ import annotations

import numpy as np

from .attention import _f64


def gate_projection(x, w, bias, B: int, n: int, Hq: int) -> np.ndarray:
    """x [B * n, Hm] (or [B, n, Hm]); w [Hm, 2 Hq]; bias [2 Hq] or None -> gates [2, B, n, Hq]."""
    x = _f64(x).reshape(B * n, -1)
    w = _f64(w)
    if w.shape != (x.shape[1], 2 * Hq):
        raise ValueError("w must be [Hm, 2 * Hq]")
    z = x @ w
    if bias is not None:
        z = z + _f64(bias)[None, :]
    g = 1.0 / (1.0 + np.exp(-z))                     # [B n, 2 Hq]
    return g.reshape(B, n, 2, Hq).transpose(2, 0, 1, 3).copy()
