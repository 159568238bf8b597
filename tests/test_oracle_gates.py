"""Pins of the oracle's gate projection (CPU): closed forms of sigmoid(x w + b)."""

import numpy as np

import oracle.gates as Gt


def test_zero_input_gives_sigmoid_of_the_bias():
    B, n, Hm, Hq = 2, 3, 16, 4
    bias = np.linspace(-3, 3, 2 * Hq)
    g = Gt.gate_projection(np.zeros((B * n, Hm)), np.random.default_rng(0).standard_normal((Hm, 2 * Hq)),
                           bias, B, n, Hq)
    want = 1 / (1 + np.exp(-bias))
    assert np.abs(g[0] - want[:Hq]).max() < 1e-15 and np.abs(g[1] - want[Hq:]).max() < 1e-15
    assert np.abs(Gt.gate_projection(np.zeros((B * n, Hm)), np.ones((Hm, 2 * Hq)), None, B, n, Hq)
                  - 0.5).max() == 0


def test_one_hot_input_picks_a_row_of_w_and_layout():
    B, n, Hm, Hq = 1, 4, 8, 2
    w = np.arange(Hm * 2 * Hq, dtype=np.float64).reshape(Hm, 2 * Hq) / 10 - 1.5
    x = np.zeros((B * n, Hm))
    for i in range(n):
        x[i, 2 * i] = 1.0
    g = Gt.gate_projection(x, w, None, B, n, Hq)
    for i in range(n):
        for path in range(2):
            for h in range(Hq):
                assert g[path, 0, i, h] == 1 / (1 + np.exp(-w[2 * i, path * Hq + h]))


def test_reflection():
    r = np.random.default_rng(1)
    B, n, Hm, Hq = 2, 5, 12, 3
    x, w, b = r.standard_normal((B * n, Hm)), r.standard_normal((Hm, 2 * Hq)), r.standard_normal(2 * Hq)
    g = Gt.gate_projection(x, w, b, B, n, Hq)
    assert np.abs(Gt.gate_projection(x, -w, -b, B, n, Hq) - (1 - g)).max() < 1e-15
